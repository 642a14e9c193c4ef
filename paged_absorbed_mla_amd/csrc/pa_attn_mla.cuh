// Read phase for wide latent rows (head sizes up to 576 / value sizes up to
// 512, the DeepSeek-V3 absorbed-MLA shape) on gfx950.
//
// Semantics are those of attn_kernel (pa_attn.cuh): docs.rs page
// "onnx-runtime-ep-cuda src/kernels/paged_attention.rs", "LATENT semantics",
// read phase (device function attn_impl).
//
// Design. One workgroup of four waves (one per SIMD, 512 registers each) owns a
// 128-row query tile (row = token_in_sequence * H + head) and walks a
// contiguous range of 32-key KV tiles:
//   * Each wave owns 32 query rows for both products, so probabilities never
//     leave registers: S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16
//     (tile_compute in pa_attn.cuh). The query (all HSP channels, 144
//     registers) and the output accumulators (256 registers) stay resident
//     for the whole piece.
//   * The query is loaded straight into MFMA fragment registers; its rotary
//     channels come already rotated from the schedule launch (a pre-pass over
//     the T x H query rows that writes them to the workspace), so the whole
//     query of a piece arrives in one batch of loads.
//   * KV tiles (32 latent rows, HSP channels, 36 KB) are copied from the paged
//     cache into four LDS buffers with direct global->LDS loads; up to three
//     tiles are in flight while one is computed. Wave w copies keys
//     [8 w, 8 w + 8) of every tile (one cache block, one scalar block-table
//     read, nine 1 KB copy instructions). Keys outside the piece's range and
//     channels >= head_size land as zeros (buffer loads past the descriptor's
//     range), so masked probabilities never meet non-finite cache values.
//   * One barrier per tile, ordering LDS only: each wave first waits for its
//     own copies of the tile (vmcnt), so after the barrier the tile is
//     complete and the buffer computed in the previous iteration is free.
//   * The first KV tiles of a piece are issued right after the query loads and
//     land while RoPE runs.
#pragma once

#include "pa_attn.cuh"

namespace pa {

// Fragment prefetch depths of the tile loop (K fragments for QK, V^T
// fragments for PV), bounded by the VGPRs left beside the resident query.
#ifndef PA_MLA_QPF
#define PA_MLA_QPF 4
#endif
#ifndef PA_MLA_VPF
#define PA_MLA_VPF 3
#endif
// LDS row layout of a staged tile: PA_MLA_PAD = 1 pads every latent row by one
// 16-byte chunk (no swizzle); 0 keeps rows dense with an XOR chunk swizzle.
#ifndef PA_MLA_SM_AFTER
#define PA_MLA_SM_AFTER 0
#endif
#ifndef PA_MLA_PAD
#define PA_MLA_PAD 0
#endif
// XOR chunk swizzle of a staged latent row: chunk c of row r sits at
// position c ^ mla_swizzle(r). Bit 2 comes from row bit 1 and bits 1..0 from
// row bits 3..2, so both LDS read patterns are free of bank conflicts (64
// banks of 4 bytes; LDS rows are 1152 bytes, an odd multiple of 128): the
// 16-lane groups of the K reads (16 consecutive rows, one chunk) and the
// 32-lane halves of the transposing V reads (4 rows x 4 aligned chunks).
__device__ __forceinline__ int mla_swizzle(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }

template <int HSP>
struct MlaLds {
  static constexpr int CPR = HSP / 8;                   // 16-byte chunks of a latent row
  static constexpr int RCH = CPR + PA_MLA_PAD;          // 16-byte chunks per LDS row
  static constexpr int ROWB = RCH * 16;                 // bytes per LDS row
  static __device__ __forceinline__ int swz(int row) { return PA_MLA_PAD ? 0 : mla_swizzle(row); }
};


// PV MFMA with the accumulator pinned to AGPRs: O^T (VHSP x 32 rows float32,
// 256 registers for 512 channels) lives in the accumulation registers for the
// whole piece while S, P, the query and the fragments use VGPRs (the kernel's
// other MFMAs are built in the VGPR form). Being inline assembly, these MFMAs
// are invisible to the compiler's hazard checks, so the kernel covers them:
// s_nop before the first PV MFMA of a tile (VALU writes of P, read as SrcB)
// and after the last one of a pass (accumulators read by VALU / stores).
// Back-to-back accumulation into the same registers needs no wait states.
template <typename DT> struct PvMfma;
template <> struct PvMfma<BF16> {
  static __device__ __forceinline__ void run(f32x16_t& acc, u32x4_t a, u32x4_t b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  }
  // acc = 0 (0 x 0 + 0), defined in AGPRs like every other value of acc.
  static __device__ __forceinline__ void zero(f32x16_t& acc, u32x4_t z) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc) : "v"(z));
  }
};
template <> struct PvMfma<F16> {
  static __device__ __forceinline__ void run(f32x16_t& acc, u32x4_t a, u32x4_t b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  }
  static __device__ __forceinline__ void zero(f32x16_t& acc, u32x4_t z) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %1, 0" : "=a"(acc) : "v"(z));
  }
};

// ds_write_b128 of four accumulation registers at LDS address addr + OFF
// (completion is awaited with lgkmcnt(0), e.g. by lds_barrier()).
template <int OFF>
__device__ __forceinline__ void ds_write_b128_acc(uint32_t addr, f32x4_t v) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset is 16 bits");
  asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(addr), "a"(v), "n"(OFF) : "memory");
}

// One 16-byte-per-lane direct global->LDS copy: lane l's 16 bytes at buffer
// offset voff land at LDS address lds_base + 16 l. Issued as inline assembly
// so that the compiler does not see an LDS write it cannot order: it would
// otherwise drain every in-flight copy (vmcnt(0)) before the next LDS read.
// The caller orders copies against LDS reads with explicit vmcnt waits and a
// barrier. `rsrc` is a raw buffer descriptor (loads past its size read zeros).
__device__ __forceinline__ void copy16_to_lds(uint32_t lds_base, uint32_t voff, u32x4_t rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds_base), "v"(voff), "s"(rsrc) : "memory", "m0");
}

// Raw buffer descriptor words over `bytes` bytes at `base` (stride 0, the same
// descriptor make_rsrc builds).
__device__ __forceinline__ u32x4_t rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}

// s_waitcnt lgkmcnt(N) that also passes `v` through, so every use of `v`
// (an LDS read issued by inline assembly, invisible to the compiler's own
// waits) is ordered after the wait.
template <int N>
__device__ __forceinline__ u32x4_t lgkm_wait_v(u32x4_t v) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(N));
  return v;
}

// rsrc_words for a wave-uniform base: the words are forced into SGPRs.
__device__ __forceinline__ u32x4_t rsrc_words_u(const void* base, uint32_t bytes) {
  u32x4_t r = rsrc_words(base, bytes);
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = __builtin_amdgcn_readfirstlane(r[k]);
  return r;
}

// 16-byte buffer load at byte offset voff through descriptor words `rsrc`
// (offsets past the descriptor's size read zeros).
__device__ __forceinline__ u32x4_t buffer_load_b128(u32x4_t rsrc, uint32_t voff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
      __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)rsrc[1] << 32) | rsrc[0]), (short)0, (int)rsrc[2],
                                        (int)rsrc[3]), voff, 0, 0));
}

// Value of lane l ^ 32 combined with lane l's own by max: one VALU lane swap
// (v_permlane32_swap), no LDS round trip.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// State one wave carries across the KV tiles of a piece.
template <int HSP, int VHSP>
struct MlaState {
  static constexpr int NKS = HSP / 16;
  static constexpr int NMT = VHSP / 32;
  u32x4_t qf[NKS];      // query rows as MFMA B fragments (k-step s: channels 16 s + 8 hi .. + 8)
  f32x16_t o[NMT];      // O^T accumulators, 32-channel blocks
  float m_ref;          // row's fixed reference (log2 units): -inf until its first visible key
  float m_seen;         // row's running maximum score (log2 units)
  float l_run;          // partial denominator sum of 2^(s - m_ref) over this lane's keys
  bool ovf;             // some score exceeded m_ref by more than the storage type allows
};

// Largest excess of a score over the reference (log2 units) for which the
// probability 2^(s - m_ref) still fits the MFMA input type and the float32
// sums: 2^15 < 65504 for float16; 2^64 for bfloat16 (8-bit exponent).
template <typename DT> struct PRange;
template <> struct PRange<BF16> { static constexpr float value = 64.0f; };
template <> struct PRange<F16> { static constexpr float value = 15.0f; };

// ---- Tile steps of the software-pipelined loop ----
// Iteration t queues the QK MFMAs of tile t (mla_qk), then runs the PV MFMAs
// of tile t - 1 with the softmax of tile t interleaved between them
// (mla_pv_softmax): the softmax never touches the accumulators (fixed
// reference), so it overlaps the matrix pipe's work instead of idling it.

// S^T = K Q^T for one 32-key tile at LDS address L. A = 32 keys x 16 channels
// (row l32, chunk 2 s + hi; chunks 8 apart share the swizzle, so the address
// is kaddr[s & 3] + 128 (s >> 2)). The reads run QPF k-steps ahead and each
// MFMA waits only for its own read. The LOADS copy instructions of a later
// tile (`copy`) are spread over the steps, one every NKS / LOADS MFMAs.
template <typename DT, int HSP, int LOADS, typename Copy>
__device__ __forceinline__ f32x16_t mla_qk(const u32x4_t* qf, uint32_t L, const uint32_t (&kaddr)[4], Copy&& copy) {
  constexpr int NKS = HSP / 16;
  constexpr int QPF = PA_MLA_QPF;
  constexpr int CSTRIDE = NKS / LOADS;
  static_assert(CSTRIDE >= 1, "copy slots");
  f32x16_t sacc = f32x16_t{};
  u32x4_t ka[QPF];
  static_for<0, QPF>([&](auto S) {
    constexpr int s = decltype(S)::value;
    ka[s] = ds_read_b128_asm<(s >> 2) * 128>(L + kaddr[s & 3]);
  });
  static_for<0, NKS>([&](auto S) {
    constexpr int s = decltype(S)::value;
    constexpr int newer = (NKS - 1 - s) < (QPF - 1) ? (NKS - 1 - s) : (QPF - 1);
    const u32x4_t cur = lgkm_wait_v<newer>(ka[s % QPF]);
    sacc = DT::mfma32(cur, qf[s], sacc);
    if constexpr (s + QPF < NKS) ka[s % QPF] = ds_read_b128_asm<((s + QPF) >> 2) * 128>(L + kaddr[(s + QPF) & 3]);
    if constexpr (s % CSTRIDE == CSTRIDE - 1 && s / CSTRIDE < LOADS) copy(std::integral_constant<int, s / CSTRIDE>{});
  });
  return sacc;
}

// O^T += V^T P^T for the tile at LDS address Lv with probabilities pf_in
// (DO_PV), and the softmax of the scores `sacc` of the tile at key0 into
// pf_out (DO_SM), its steps placed between the PV MFMAs.
//   PV: A = 32 channels x 16 keys via two transposing reads (step n: k-step
//   n / NMT, channel block n % NMT); k-index 8 g + e of lane group g is key
//   4 g + (e & 3) + 8 (e >> 2), the key order of the S^T accumulator, so P^T
//   comes straight from the softmax registers.
//   Softmax: lane holds row l32 and keys hi*4 + (e & 3) + 8 (e >> 2) of the
//   tile. Fixed reference: the row's first tile with a visible key sets m_ref
//   (the accumulators are still zero then, so nothing needs rescaling); later
//   probabilities are 2^(s - m_ref), which may exceed 1, numerator and
//   denominator share the reference, so the quotient is unchanged. A score
//   more than PRange above the reference flags the piece for a second pass
//   with the row's exact maximum as reference (the accumulators are never
//   rescaled in place).
template <typename DT, int HSP, int VHSP, bool DO_PV, bool DO_SM>
__device__ __forceinline__ void mla_pv_softmax(MlaState<HSP, VHSP>& st, uint32_t Lv, const uint32_t (&vaddr)[4],
                                               const u32x4_t (&pf_in)[2], f32x16_t sacc, int key0, int pos,
                                               int lo_row, bool softcap_on, const AttnParams& p, u32x4_t (&pf_out)[2]) {
  constexpr int CPR = HSP / 8;
  constexpr int NMT = VHSP / 32;
  constexpr int VPF = PA_MLA_VPF;
  constexpr int VSTEPS = 2 * NMT;
  const int lane = threadIdx.x & 63;
  const int hi = lane >> 5;

  auto v_frag = [&](auto NN) -> u32x4_t {
    constexpr int n = decltype(NN)::value;
    constexpr int k2 = n / NMT, mt = n % NMT;
    constexpr int off = k2 * 16 * MlaLds<HSP>::ROWB + (mt >> 1) * 128;
    const u32x2_t r0 = ds_read_tr16_b64_asm<off>(Lv + vaddr[mt & 1]);
    const u32x2_t r1 = ds_read_tr16_b64_asm<off>(Lv + vaddr[2 + (mt & 1)]);
    return u32x4_t{r0[0], r0[1], r1[0], r1[1]};
  };
  u32x4_t va[VPF];
  if constexpr (DO_PV) {
    static_for<0, VPF>([&](auto N) { va[decltype(N)::value] = v_frag(N); });
    // VALU writes of P (SrcB) precede the first PV MFMA.
    asm volatile("s_nop 4");
  }

  // Softmax state shared by the chunks below.
  float tmax = -INFINITY, m_use = 0.0f, psum = 0.0f;
  float pv[16];
  const bool full_tile = key0 >= lo_row && key0 + 31 <= pos;
  // Chunk c of the softmax; chunks are ordered by data dependence.
  auto sm_chunk = [&](auto C) {
    constexpr int c = decltype(C)::value;
    if constexpr (c == 0) {
      // scale (and softcap) into log2 units
      if (softcap_on) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[e] = softcap_log2(sacc[e], p.scale, p.softcap, p.softcap_inv);
      } else {
        sacc *= p.scale_log2;
      }
    } else if constexpr (c == 1) {
      // mask and tile max
      if (full_tile) {
#pragma unroll
        for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, sacc[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int j = key0 + hi * 4 + (e & 3) + 8 * (e >> 2);
          const float v = (j <= pos && j >= lo_row) ? sacc[e] : -INFINITY;
          sacc[e] = v;
          tmax = fmaxf(tmax, v);
        }
      }
    } else if constexpr (c == 2) {
      tmax = max_xor32(tmax);
      st.m_seen = fmaxf(st.m_seen, tmax);
      if (st.m_ref == -INFINITY) st.m_ref = tmax;
      st.ovf |= tmax > st.m_ref + PRange<DT>::value;
      m_use = (st.m_ref == -INFINITY) ? 0.0f : st.m_ref;
    } else if constexpr (c >= 3 && c < 11) {
      constexpr int k = c - 3;   // probabilities of elements 2k, 2k + 1
      pv[2 * k] = fast_exp2(sacc[2 * k] - m_use);
      pv[2 * k + 1] = fast_exp2(sacc[2 * k + 1] - m_use);
      psum += pv[2 * k] + pv[2 * k + 1];
    } else if constexpr (c == 11) {
      float lo[8], hi8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lo[e] = pv[e];
        hi8[e] = pv[8 + e];
      }
      pf_out[0] = pack8<DT>(lo);
      pf_out[1] = pack8<DT>(hi8);
      st.l_run += psum;
    }
  };
  constexpr int NCHUNK = 12;

  if constexpr (DO_PV) {
    // Softmax chunk c runs after PV step 2 c + 1 (all chunks fit in the steps).
    static_assert(2 * NCHUNK <= VSTEPS, "softmax chunks fit between the PV steps");
    static_for<0, VSTEPS>([&](auto N) {
      constexpr int n = decltype(N)::value;
      constexpr int newer = (VSTEPS - 1 - n) < (VPF - 1) ? (VSTEPS - 1 - n) : (VPF - 1);
      const u32x4_t cur = lgkm_wait_v<2 * newer>(va[n % VPF]);
      PvMfma<DT>::run(st.o[n % NMT], cur, pf_in[n / NMT]);
      if constexpr (n + VPF < VSTEPS) va[n % VPF] = v_frag(std::integral_constant<int, n + VPF>{});
#if PA_MLA_SM_AFTER == 0
      if constexpr (DO_SM && (n % 2 == 1) && (n / 2 < NCHUNK)) sm_chunk(std::integral_constant<int, n / 2>{});
      __builtin_amdgcn_sched_barrier(0);
#endif
    });
#if PA_MLA_SM_AFTER
    if constexpr (DO_SM) static_for<0, NCHUNK>([&](auto C) { sm_chunk(C); });
#endif
  } else if constexpr (DO_SM) {
    static_for<0, NCHUNK>([&](auto C) { sm_chunk(C); });
  }
}

template <typename DT, int HSP, int VHSP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void attn_mla_kernel(AttnParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NW = 4;
  constexpr int KT = 32;
  constexpr int NB = 4;                   // LDS tile buffers
  constexpr int RW = NW * 32;             // rows of a query tile
  constexpr int CPR = HSP / 8;            // 16-byte chunks per LDS row
  constexpr int NKS = HSP / 16;           // 16-channel k-steps of QK
  constexpr int NMT = VHSP / 32;          // 32-channel output blocks
  constexpr int KW = KT / NW;             // keys each wave copies per tile
  constexpr int SLOTS = KW * CPR;         // 16-byte copies per wave per tile
  constexpr int LOADS = SLOTS / 64;       // copy instructions per wave per tile
  constexpr int BUF_BYTES = KT * CPR * 16;
  constexpr int LDS_BYTES = NB * BUF_BYTES;
  static_assert(SLOTS % 64 == 0, "whole copy instructions");
  static_assert(HSP % 64 == 0 && VHSP % 32 == 0 && VHSP <= HSP, "head sizes");
  static_assert((NB - 3) * LOADS <= 63, "vmcnt range");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(KW * HSP * 2 <= 0xFFFF, "16-bit copy offsets");
  __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[LDS_BYTES];

  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int wr = range_of_block();
  int u = ld_uniform(p.wg_range + wr);
  const int u_end = ld_uniform(p.wg_range + wr + 1);
  if (u >= u_end) return;
  int i = ld_uniform(p.wg_tile + wr);   // query tile holding unit u
  const bool softcap_on = p.softcap > 0.0f;

  // Copy slot sl = it * 64 + lane of this wave is LDS row 8 w + sl / CPR,
  // position sl % CPR, which holds chunk (sl % CPR) ^ swizzle(row). Its source
  // is byte off(it) of the wave's KW cache rows; two 16-bit offsets per
  // register. Chunks at channels >= hs get 0xFFFF, past the descriptor's range.
  constexpr int NOFF = (LOADS + 1) / 2;
  uint32_t load_off2[NOFF];
#pragma unroll
  for (int k2 = 0; k2 < NOFF; ++k2) load_off2[k2] = 0xFFFFFFFFu;
#pragma unroll
  for (int it = 0; it < LOADS; ++it) {
    const int sl = it * 64 + lane;
    const int k = sl / CPR;
    const int lc = (sl - k * CPR) ^ mla_swizzle(w * KW + k);
    const uint32_t off = lc * 8 < p.hs ? (uint32_t)((k * p.hs + lc * 8) * 2) : 0xFFFFu;
    const int sh = (it & 1) * 16;
    load_off2[it >> 1] = (load_off2[it >> 1] & ~(0xFFFFu << sh)) | (off << sh);
  }

  while (u < u_end) {
    const MTile t = ld_uniform_tile(p.mt + i);
    const int next0 = ld_uniform(&p.mt[i + 1].unit0);
    const int ua = u;
    const int ub = min(u_end, next0);
    const int tile_a = t.kv_lo / KT + (ua - t.unit0);
    const int tile_b = tile_a + (ub - ua);
    const bool whole = (ua == t.unit0) && (ub == next0);
    const int b = t.b;
    const int cum_b = ld_uniform(p.cumseq + b);
    const int past_b = ld_uniform(p.past + b);

    // This lane's query row (rows past the tile read row 0 of the tile and are
    // never stored; each row's softmax and output column are independent).
    const int rloc = w * 32 + l32;
    const bool row_ok = rloc < t.nrows;
    const int R = t.row0 + (row_ok ? rloc : 0);
    const int tq = R / p.H;
    const int h = R - tq * p.H;
    const int pos = past_b + tq;
    const int lo_row = p.window >= 0 ? max(0, pos - p.window) : 0;
    const int64_t qrow = (int64_t)(cum_b + tq) * p.H + h;

    // Query fragments: k-step s holds channels 16 s + 8 hi .. + 8 of the row.
    // The wave's 32 rows are consecutive in `query`; one wave-uniform buffer
    // descriptor starts at its first row and each lane's row and chunk go in
    // the per-lane offset (chunks past hs take an out-of-range offset and read
    // zeros).
    MlaState<HSP, VHSP> st;
    const int64_t wrow0 = (int64_t)cum_b * p.H + t.row0 + 32 * w;   // first query row of the wave
    {
      const u32x4_t qrs = rsrc_words_u(p.query + wrow0 * p.hs, (uint32_t)(32 * p.hs * 2));
      const int ln = opaque_lane();
      const int lr = (32 * w + (ln & 31)) < t.nrows ? (ln & 31) : 0;
      const uint32_t qbase = (uint32_t)(lr * p.hs * 2);
      const int h8 = (ln >> 5) * 8;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const int c0 = 16 * s + h8;
        st.qf[s] = buffer_load_b128(qrs, c0 < p.hs ? qbase + (uint32_t)(c0 * 2) : kOutOfRange);
      }
      // Rotary chunks come from the RoPE'd copy the schedule launch wrote
      // (qrot, rd channels per row); the test on the k-step is uniform and the
      // geometry is opaque so nothing is hoisted out of the piece loop.
      if (p.do_rotary) {
        int ro = p.ro, rd = p.rd;
        asm volatile("" : "+s"(ro), "+s"(rd));
        const u32x4_t rrs = rsrc_words_u(p.qrot + wrow0 * rd, (uint32_t)(32 * rd * 2));
        const uint32_t rbase = (uint32_t)(lr * rd * 2);
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
          if (16 * s + 16 > ro && 16 * s < ro + rd) {
            const int c0 = 16 * s + h8;
            if (c0 >= ro && c0 < ro + rd) st.qf[s] = buffer_load_b128(rrs, rbase + (uint32_t)((c0 - ro) * 2));
          }
        }
      }
    }

    // The query has landed before any tile copy is issued (the compiler's own
    // wait for these loads would otherwise sit inside the tile loop and drain
    // the copy pipeline on every tile): vmcnt(0), expcnt/lgkmcnt unconstrained.
    __builtin_amdgcn_s_waitcnt(0x0F70);

    // Copy KV tile `tile` into LDS buffer `bufi`: exactly LOADS copy
    // instructions per wave (vmcnt counts them).
    // Block id of the cache block holding this wave's keys of `tile`.
    auto block_of = [&](int tile) -> int {
      const int kw0 = tile * KT + w * KW;
      return ld_uniform(p.bt + (int64_t)b * p.MB + min(kw0 >> p.bs_log2, p.MB - 1));
    };
    // A planned tile copy: descriptor over the wave's KW cache rows, LDS
    // destination, and whether every key of the slice is in range.
    struct CopyPlan {
      u32x4_t rsrc;
      uint32_t dst0;
      int kw0;
      bool full;
    };
    auto plan = [&](int tile, int bufi, int blk_raw) -> CopyPlan {
      CopyPlan c;
      c.kw0 = tile * KT + w * KW;
      const int blk = clamp_block(blk_raw, p.nblk);
      const uint16_t* rows = p.cache + (((int64_t)blk << p.bs_log2) + (c.kw0 & ((1 << p.bs_log2) - 1))) * p.hs;
      c.rsrc = rsrc_words_u(rows, (uint32_t)(KW * p.hs * 2));
      c.dst0 = lds_addr(lds_raw) + (uint32_t)(bufi * BUF_BYTES + w * SLOTS * 16);
      c.full = c.kw0 >= t.kv_lo && c.kw0 + KW <= t.kv_hi;
      return c;
    };
    // Copy instruction `it` of a planned tile (LDS slots it*64 .. it*64+63 of
    // the wave's slice). Exactly LOADS of them per tile and wave (vmcnt counts
    // them).
    auto copy_one = [&](const CopyPlan& c, int it) {
      uint32_t o2 = load_off2[it >> 1];
      asm volatile("" : "+v"(o2));
      uint32_t off = (o2 >> ((it & 1) * 16)) & 0xFFFFu;
      if (!c.full) {
        const int j = c.kw0 + (it * 64 + opaque_lane()) / CPR;
        off = (j >= t.kv_lo && j < t.kv_hi) ? off : kOutOfRange;
      }
      copy16_to_lds(c.dst0 + it * 64 * 16, off, c.rsrc);
    };
    auto issue = [&](int tile, int bufi, int blk_raw) {
      const CopyPlan c = plan(tile, bufi, blk_raw);
#pragma unroll
      for (int it = 0; it < LOADS; ++it) copy_one(c, it);
    };

    // LDS fragment addresses of this lane relative to a tile buffer.
    // K (QK A operand): row l32, chunk 2 s + hi; four bases cover s & 3.
    uint32_t kaddr[4], vaddr[4];
    {
      const int ln = opaque_lane();
      const int r32 = ln & 31, h1 = ln >> 5;
      const int swk = mla_swizzle(r32);
#pragma unroll
      for (int r = 0; r < 4; ++r) kaddr[r] = r32 * CPR * 16 + (((2 * r + h1) ^ swk) << 4);
      // V^T (PV A operand), transposing reads: lane (g, jj, cq) supplies row
      // 4 (g >> 1) + jj (and + 8) and channel quad cq of its 16-lane group.
      const int g = ln >> 4, jj = (ln & 15) >> 2, cq = ln & 3;
      const int k0b = (g >> 1) * 4 + jj;
      const int sw0 = mla_swizzle(k0b), sw1 = mla_swizzle(k0b + 8);
      const int lcb = 2 * (g & 1) + (cq >> 1);
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        vaddr[par] = k0b * CPR * 16 + (((4 * par + lcb) ^ sw0) << 4) + (cq & 1) * 8;
        vaddr[2 + par] = (k0b + 8) * CPR * 16 + (((4 * par + lcb) ^ sw1) << 4) + (cq & 1) * 8;
      }
    }
    const uint32_t lds0 = lds_addr(lds_raw);

    // One pass normally; a second one (reference = the rows' exact maxima from
    // the first) only when some score overflowed the first pass's reference.
    st.m_ref = -INFINITY;
    st.m_seen = -INFINITY;
    for (int pass = 0; pass < 2; ++pass) {
      // Software pipeline over the piece's tiles (buffer of tile k: (k - tile_a)
      // % NB). Iteration tt queues QK(tt) with the copies of tile tt + 2
      // interleaved, then runs PV(tt - 1) with the softmax of tt between its
      // MFMAs. Live buffers in iteration tt: tt (K), tt - 1 (V); tiles tt + 1
      // and tt + 2 are in flight; tt + 2 reuses the buffer of tt - 2, whose V
      // every wave consumed before this iteration's barrier.
      constexpr int AHEAD = NB - 2;   // tiles in flight beyond the current one
#pragma unroll
      for (int k = 0; k < AHEAD; ++k)
        if (tile_a + k < tile_b) issue(tile_a + k, k, block_of(tile_a + k));
      {
        const u32x4_t z = {0u, 0u, 0u, 0u};
        asm volatile("s_nop 4");   // VALU write of z precedes its use as SrcA/B
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) PvMfma<DT>::zero(st.o[mt], z);
      }
      st.l_run = 0.0f;
      st.ovf = false;

      int blk_next = block_of(min(tile_a + AHEAD, tile_b - 1));
      const int rpos = row_ok ? pos : -1;
      // One pipeline step: wait for tile tt, queue QK(tt) with the copies of
      // tile tt + AHEAD, then (PV(tt - 1) and) the softmax of tt.
      auto qk_step = [&](int tt) -> f32x16_t {
        vm_wait_tiles<LOADS, AHEAD - 1>(min(AHEAD - 1, tile_b - 1 - tt));
        lds_barrier();   // tile tt complete; every wave is done with tile tt - 2
        // Copies of tile tt + AHEAD go out during the QK MFMAs of tile tt; their
        // block id was read one iteration earlier.
        const int blk_cur = blk_next;
        blk_next = block_of(min(tt + AHEAD + 1, tile_b - 1));
        const bool more = tt + AHEAD < tile_b;
        const CopyPlan cp = plan(tt + AHEAD, (tt + AHEAD - tile_a) % NB, blk_cur);
        return mla_qk<DT, HSP, LOADS>(st.qf, lds0 + ((tt - tile_a) % NB) * BUF_BYTES, kaddr, [&](auto IT) {
          if (more) copy_one(cp, decltype(IT)::value);
        });
      };
      u32x4_t pf[2];
      {
        const f32x16_t sacc = qk_step(tile_a);
        mla_pv_softmax<DT, HSP, VHSP, false, true>(st, 0, vaddr, pf, sacc, tile_a * KT, rpos, lo_row, softcap_on, p,
                                                   pf);
      }
      for (int tt = tile_a + 1; tt < tile_b; ++tt) {
        const f32x16_t sacc = qk_step(tt);
        const uint32_t Lv = lds0 + ((tt - 1 - tile_a) % NB) * BUF_BYTES;
        u32x4_t pf_new[2];
        mla_pv_softmax<DT, HSP, VHSP, true, true>(st, Lv, vaddr, pf, sacc, tt * KT, rpos, lo_row, softcap_on, p,
                                                  pf_new);
        pf[0] = pf_new[0];
        pf[1] = pf_new[1];
      }
      // PV of the last tile (its buffer is still resident).
      mla_pv_softmax<DT, HSP, VHSP, true, false>(st, lds0 + ((tile_b - 1 - tile_a) % NB) * BUF_BYTES, vaddr, pf,
                                                 f32x16_t{}, 0, 0, 0, false, p, pf);
      // Whole-workgroup vote on a second pass (the tile buffers are free once
      // every wave passed the barrier; the flags sit in the first buffer).
      lds_barrier();
      int* const vote = (int*)lds_raw;
      if (lane == 0) vote[w] = __any(st.ovf) ? 1 : 0;
      lds_barrier();
      const int again = vote[0] | vote[1] | vote[2] | vote[3];
      lds_barrier();     // votes read before the buffers are reused
      if (!again) break;
      st.m_ref = st.m_seen;
    }
    // PV accumulators are read below (LDS writes from AGPRs).
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

    // Epilogue through LDS (the tile buffers are free): O^T of all rows is
    // staged as float32 rows, half of the value channels at a time, written
    // straight from the accumulation registers, then every thread normalises
    // (whole tile) or copies (partial result) 8 consecutive channels of a row
    // with coalesced stores. Rows are padded by 16 bytes against bank conflicts.
    const float l_tot = st.l_run + __shfl_xor(st.l_run, 32);
    constexpr int HALF = VHSP / 2;
    constexpr int ORS = HALF + 4;                          // floats per staged row
    constexpr int C8 = HALF / 8;                           // 8-channel groups per staged row
    static_assert((RW * ORS + 2 * RW) * 4 <= LDS_BYTES, "epilogue staging fits the tile buffers");
    static_assert((NMT / 2) % 1 == 0 && HALF % 32 == 0, "whole accumulator blocks per half");
    float* const ost = (float*)lds_raw;
    float* const rowl = ost + RW * ORS;                    // [RW] denominators
    if (hi == 0) rowl[rloc] = l_tot;
    const int64_t slot = whole ? 0 : (int64_t)t.part_base + (wr - t.w_first);
    if (!whole && hi == 0 && row_ok) {
      float* ml = p.part_ml + (slot * RW + rloc) * 2;
      ml[0] = st.m_ref;
      ml[1] = l_tot;
    }
    const uint32_t wbase = lds_addr(ost) + (uint32_t)((rloc * ORS + 4 * hi) * 4);
    const int64_t orow0 = (int64_t)cum_b * p.H + t.row0;  // output row of local row 0
    static_for<0, 2>([&](auto HF) {
      constexpr int half = decltype(HF)::value;
      static_for<0, 2 * NMT>([&](auto K) {
        constexpr int mloc = decltype(K)::value / 4;
        constexpr int j = decltype(K)::value % 4;
        constexpr int mt = half * (NMT / 2) + mloc;
        const f32x4_t part = __builtin_shufflevector(st.o[mt], st.o[mt], 4 * j, 4 * j + 1, 4 * j + 2, 4 * j + 3);
        ds_write_b128_acc<(32 * mloc + 8 * j) * 4>(wbase, part);
      });
      lds_barrier();     // staged half visible (the asm writes are waited for by lgkmcnt(0))
      for (int idx = (int)threadIdx.x; idx < RW * C8; idx += NW * 64) {
        const int r = idx / C8;
        const int c = (idx - r * C8) * 8;
        const int cg = half * HALF + c;                    // value channel
        if (r >= t.nrows || cg >= p.vhs) continue;
        const f32x4_t v0 = *(const f32x4_t*)(ost + r * ORS + c);
        const f32x4_t v1 = *(const f32x4_t*)(ost + r * ORS + c + 4);
        if (whole) {
          const float lr = rowl[r];
          const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
          const float x[8] = {v0[0] * inv, v0[1] * inv, v0[2] * inv, v0[3] * inv,
                              v1[0] * inv, v1[1] * inv, v1[2] * inv, v1[3] * inv};
          uint16_t* dst = p.out + (orow0 + r) * p.vhs + cg;
          if (cg + 8 <= p.vhs && (p.vhs & 7) == 0) {
            *(u32x4_t*)dst = pack8<DT>(x);
          } else {
            for (int k = 0; k < 8 && cg + k < p.vhs; ++k) dst[k] = (uint16_t)DT::from_f32(x[k]);
          }
        } else {
          float* dst = p.part_acc + slot * p.part_slot + (int64_t)r * p.part_row + cg;
          *(f32x4_t*)dst = v0;
          *(f32x4_t*)(dst + 4) = v1;
        }
      }
      lds_barrier();     // staging area free again
    });
    u = ub;
    ++i;
  }
#endif  // __HIP_DEVICE_COMPILE__
}

}  // namespace pa

#define PA_DEFINE_ATTN_MLA_INSTANCE(DT, DTN, HSP, VHSP)                                                 \
  namespace pa {                                                                                        \
  hipError_t PA_ATTN_FN(DTN, HSP, VHSP, 4, 32, occ)(int* n) {                                           \
    void (*fn)(AttnParams) = attn_mla_kernel<DT, HSP, VHSP>;                                            \
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, reinterpret_cast<const void*>(fn), 256, 0);  \
  }                                                                                                     \
  hipError_t PA_ATTN_FN(DTN, HSP, VHSP, 4, 32, launch)(const AttnParams& p, int grid, bool combine,      \
                                                       int cgrid, hipStream_t s, const hipEvent_t* ev) { \
    hipError_t e = ev ? hipEventRecord(ev[0], s) : hipSuccess;                                          \
    if (e != hipSuccess) return e;                                                                      \
    attn_mla_kernel<DT, HSP, VHSP><<<grid, 256, 0, s>>>(p);                                             \
    e = hipGetLastError();                                                                              \
    if (e == hipSuccess && ev) e = hipEventRecord(ev[1], s);                                            \
    if (e != hipSuccess || !combine) return e;                                                          \
    combine_kernel<DT, VHSP, 128><<<dim3(cgrid, 128 / kCombineRows), 256, 0, s>>>(p);                   \
    return hipGetLastError();                                                                           \
  }                                                                                                     \
  }
