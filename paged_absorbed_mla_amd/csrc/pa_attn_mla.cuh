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
//   * QK, row split: each wave keeps its 32 query rows (all HSP channels, 144
//     registers) resident as MFMA fragments and forms S^T = K Q^T for them on
//     v_mfma_f32_32x32x16. The query comes from a copy the schedule launch
//     writes in fragment order with RoPE applied, so each load instruction
//     reads one contiguous run.
//   * PV, channel split: wave w accumulates O^T for all 128 rows but only value
//     channels [128 w, 128 w + 128) (256 accumulator registers). Each wave
//     writes its rows' probabilities of a tile once to a double-buffered LDS
//     area in the S^T accumulator layout; every wave reads all of them and a
//     quarter of V with transposing reads.
//   * Fixed-reference softmax: a row's first tile with a visible key fixes
//     its reference; the accumulators are never rescaled, and a score beyond
//     the probability type's range above the reference sends the piece
//     through a second pass with exact maxima.
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
//   * The first two KV tiles of a piece are issued before the query loads, so
//     their latencies overlap.
//   * Epilogue through LDS with coalesced stores: the output rows of a whole
//     query tile, or the piece's partial slot for the split-KV combine.
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

// ds_write_b128 of four VGPRs at LDS address addr + OFF (completion is
// awaited with lgkmcnt(0), e.g. by lds_barrier()).
template <int OFF>
__device__ __forceinline__ void ds_write_b128_v(uint32_t addr, u32x4_t v) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset is 16 bits");
  asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(addr), "v"(v), "n"(OFF) : "memory");
}

// s_waitcnt lgkmcnt(N) that also passes `v` through, so every use of `v`
// (an LDS read issued by inline assembly, invisible to the compiler's own
// waits) is ordered after the wait.
template <int N>
__device__ __forceinline__ u32x4_t lgkm_wait_v(u32x4_t v) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(N));
  return v;
}

// s_waitcnt lgkmcnt(N) (vmcnt and expcnt unconstrained) that no instruction
// is scheduled across. Used where the reads it waits for and their consumers
// are all inline assembly or fixed in program order, so unlike lgkm_wait_v it
// does not pretend to write the read destinations (which would make the
// compiler add a hazard wait state before the MFMA that consumes them).
template <int N>
__device__ __forceinline__ void lgkm_wait_fence() {
  static_assert(N >= 0 && N < 16, "lgkmcnt field");
  __builtin_amdgcn_s_waitcnt(0xC07F | (N << 8));
  __builtin_amdgcn_sched_barrier(0);
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

// Sum of lane l's value and lane l ^ 32's (the same swap; the two halves get
// bit-identical sums since addition commutes). Needs no lane id, unlike a
// permute, whose address the compiler would keep in a spill slot.
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// State one wave carries across the KV tiles of a piece.
template <int HSP, int VHSP>
struct MlaState {
  static constexpr int NKS = HSP / 16;
  static constexpr int NMT = VHSP / 32;
  u32x4_t qf[NKS];      // query rows as MFMA B fragments (k-step s: channels 16 s + 8 hi .. + 8)
  f32x16_t o[NMT];      // O^T accumulators: o[4 c + r] = this wave's channel block c x row block r
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
// Headroom of a reference taken from a tile where the row sees at most four
// keys (a window edge, the first keys of a sequence): the maximum of so few
// scores sits well below the row's, so with float16's narrow range the
// reference starts that many log2 units higher (the row's larger
// probabilities stay near 1, inside float16's normal range). bfloat16 needs none.
template <typename DT> struct PHead;
template <> struct PHead<BF16> { static constexpr float value = 0.0f; };
template <> struct PHead<F16> { static constexpr float value = 8.0f; };

// ---- Tile steps of the software-pipelined loop ----
// Iteration t queues the QK MFMAs of tile t (mla_qk), then runs the PV MFMAs
// of tile t - 1 with the softmax of tile t interleaved between them
// (mla_pv_softmax): the softmax never touches the accumulators (fixed
// reference), so it overlaps the matrix pipe's work instead of idling it.

// S^T = K Q^T for one 32-key tile at LDS address L. A = 32 keys x 16 channels
// (row l32, chunk 2 s + hi; chunks 8 apart share the swizzle, so the address
// is kaddr[s & 3] + 128 (s >> 2)). The reads run QPF k-steps ahead; one wait
// (in place on the two read destinations) covers the reads of k-steps s and
// s + 1, so there is one wait per two MFMAs. The LOADS copy instructions of a
// later tile (`copy`) are spread over the steps, one every NKS / LOADS MFMAs,
// and between(s) runs after MFMA s (the previous tile's softmax steps).
template <typename DT, int HSP, int LOADS, typename Copy, typename Between>
__device__ __forceinline__ f32x16_t mla_qk(const u32x4_t* qf, uint32_t L, const uint32_t (&kaddr)[4], Copy&& copy,
                                           Between&& between) {
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
  static_assert(QPF % 2 == 0 && NKS % 2 == 0, "k-steps waited for in pairs");
  static_for<0, NKS>([&](auto S) {
    constexpr int s = decltype(S)::value;
    if constexpr (s % 2 == 0) {
      // Reads issued so far: k-steps 0 .. min(s + QPF - 1, NKS - 1).
      constexpr int last = (s + QPF - 1) < (NKS - 1) ? (s + QPF - 1) : (NKS - 1);
      lgkm_wait_fence<last - (s + 1)>();
    }
    sacc = DT::mfma32(ka[s % QPF], qf[s], sacc);
    if constexpr (s + QPF < NKS) ka[s % QPF] = ds_read_b128_asm<((s + QPF) >> 2) * 128>(L + kaddr[(s + QPF) & 3]);
    if constexpr (s % CSTRIDE == CSTRIDE - 1 && s / CSTRIDE < LOADS) copy(std::integral_constant<int, s / CSTRIDE>{});
    between(S);
  });
  return sacc;
}

// Static order of the LDS reads of one PV step (32 MFMAs; MFMA n covers
// k-step ks = n / 16, the wave's channel block c = (n / 4) % 4 and row block
// r = n % 4). P fragments: the four of a k-step are read together, those of
// k-step 1 during steps 8..11. V^T fragments (two reads each): two channel
// blocks ahead. Issued before MFMA 0: P(0, 0..3), V(0, 0), V(0, 1) (8 reads).
// wait(n) is the number of LDS reads that may still be in flight when MFMA n
// issues (reads complete in order), capped at the 4-bit lgkmcnt field.
struct PvSched {
  static constexpr int kPre = 8;
  static constexpr int at(int m) {   // reads issued right after MFMA m
    return m == 8 ? 4 : ((m == 0 || m == 4 || m == 10 || m == 12 || m == 16 || m == 20) ? 2 : 0);
  }
  static constexpr int before(int n) {
    int t = kPre;
    for (int m = 0; m < n; ++m) t += at(m);
    return t;
  }
  static constexpr int endV(int ks, int c) {   // reads issued up to and including V(ks, c)
    return ks == 0 ? (c == 0 ? 6 : c == 1 ? 8 : c == 2 ? before(1) : before(5))
                   : (c == 0 ? before(8) + 2 : before(8 + 4 * c + 1));
  }
  static constexpr int endP(int ks, int r) {
    return ks == 0 ? r + 1 : (r < 2 ? before(8) + 3 + r : before(10) + r - 1);
  }
  static constexpr int wait(int n) {
    const int ks = n / 16, c = (n / 4) % 4, r = n % 4;
    const int e = endV(ks, c) > endP(ks, r) ? endV(ks, c) : endP(ks, r);
    const int w = before(n) - e;
    return w > 15 ? 15 : w;
  }
};
static_assert(PvSched::wait(0) >= 0 && PvSched::wait(16) >= 0 && PvSched::wait(31) >= 0, "read order");

// Softmax of one tile for this wave's 32 rows, in kSmChunks steps that the
// caller spreads over the MFMAs of a PV step. Lane holds row l32 and keys hi*4 + (e & 3) + 8 (e >> 2) of the tile.
// Fixed reference: the row's first tile with a visible key sets m_ref (the
// accumulators are still zero then, so nothing needs rescaling); later
// probabilities are 2^(s - m_ref), which may exceed 1, numerator and
// denominator share the reference, so the quotient is unchanged. A score more
// than PRange above the reference flags the piece for a second pass with the
// row's exact maximum as reference (the accumulators are never rescaled in
// place). full_tile (uniform): every key of the tile is visible to every
// valid row of the wave, so no per-lane mask is formed.
struct MlaSm {
  f32x16_t s;        // scores of the tile (raw when the scale is fused, else log2 units after step 0)
  float tmax, m_use, psum;
  u32x4_t pf[2];     // probabilities as PV B fragments (k-steps 0 and 1), packed as they are formed
};
constexpr int kSmChunks = 12;

template <typename DT, int HSP, int VHSP, int C>
__device__ __forceinline__ void mla_sm_chunk(MlaState<HSP, VHSP>& st, MlaSm& sm, int key0, int pos, int lo_row,
                                             bool full_tile, bool softcap_on, const AttnParams& p) {
  // Scale fused into the exponent (no softcap, scale > 0): the maximum of the
  // raw scores times the scale is the maximum logit (rounding is monotone),
  // and each probability is 2^fma(s, scale, -reference). Otherwise step 0
  // forms the logits and the multiplier is 1.
  const bool fused = !softcap_on && p.scale_log2 > 0.0f;
  if constexpr (C == 0) {
    sm.tmax = -INFINITY;
    sm.psum = 0.0f;
    if (!fused) {
      if (softcap_on) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sm.s[e] = softcap_log2(sm.s[e], p.scale, p.softcap, p.softcap_inv);
      } else {
        const float c = p.scale_log2;
#pragma unroll
        for (int e = 0; e < 16; ++e) sm.s[e] *= c;
      }
    }
  } else if constexpr (C == 1) {
    // mask (in place, only for a tile some row does not see whole) and tile max
    if (!full_tile) {
      // Lane half re-derived here (a copy kept across the tile loop would sit
      // in a spill slot).
      const int hi = fresh_lane() >> 5;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = key0 + hi * 4 + (e & 3) + 8 * (e >> 2);
        sm.s[e] = (j <= pos && j >= lo_row) ? sm.s[e] : -INFINITY;
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) sm.tmax = fmaxf(sm.tmax, sm.s[e]);
  } else if constexpr (C == 2) {
    const float tmax = fused ? max_xor32(sm.tmax) * p.scale_log2 : max_xor32(sm.tmax);
    st.m_seen = fmaxf(st.m_seen, tmax);
    if (st.m_ref == -INFINITY) {
      if constexpr (PHead<DT>::value > 0.0f) {
        const int nvis = full_tile ? 32 : min(pos, key0 + 31) - max(lo_row, key0) + 1;   // row's visible keys
        st.m_ref = tmax + (nvis <= 4 ? PHead<DT>::value : 0.0f);
      } else {
        st.m_ref = tmax;
      }
    }
    st.ovf |= tmax > st.m_ref + PRange<DT>::value;
    sm.m_use = (st.m_ref == -INFINITY) ? 0.0f : st.m_ref;
  } else if constexpr (C >= 3 && C < 11) {
    constexpr int k = C - 3;   // probabilities of elements 2k, 2k + 1 -> word k of the fragments
    const float mul = fused ? p.scale_log2 : 1.0f;
    const float p0 = fast_exp2(__builtin_fmaf(sm.s[2 * k], mul, -sm.m_use));
    const float p1 = fast_exp2(__builtin_fmaf(sm.s[2 * k + 1], mul, -sm.m_use));
    sm.pf[k >> 2][k & 3] = DT::pack2(p0, p1);
    sm.psum = DT::sum2(sm.pf[k >> 2][k & 3], sm.psum);   // the rounded pair, as the PV product sees it
  } else if constexpr (C == 11) {
    st.l_run += sm.psum;
  }
  static_assert(C < kSmChunks, "softmax steps");
}

// This wave's probabilities to the P buffer at Pb: fragment (row block w,
// k-step ks) at Pb + (2 w + ks) * 1024, lane-major.
__device__ __forceinline__ void mla_sm_store(const MlaSm& sm, uint32_t Pb) {
  const uint32_t dst = Pb + (uint32_t)(threadIdx.x >> 6) * 2048u + (uint32_t)(threadIdx.x & 63) * 16u;
  ds_write_b128_v<0>(dst, sm.pf[0]);
  ds_write_b128_v<1024>(dst, sm.pf[1]);
}

// PV step with the value channels split across the waves: O^T += V^T P^T for
// the tile at LDS address Lv, where wave w holds all 128 rows of the query
// tile and value channels [128 w, 128 w + 128). Its A operands are the V^T
// fragments of its own channel blocks only (transposing reads; the wave's
// offset is folded into vaddr) and its B operands are the four row blocks'
// probabilities P^T, which every wave wrote to the P buffer at Lp. Compared
// with every wave reading all of V for its own 32 rows, a wave reads a
// quarter of V plus 8 KB of P per tile. k-index 8 g + e of lane group g is
// key 4 g + (e & 3) + 8 (e >> 2), the key order of the S^T accumulator.
// between(n) runs after MFMA n (the next tile's softmax steps; the MFMAs leave
// issue slots for them).
template <typename DT, int HSP, int VHSP, typename Between>
__device__ __forceinline__ void mla_pv(MlaState<HSP, VHSP>& st, uint32_t Lv, const uint32_t (&vaddr)[4], uint32_t Lp,
                                       Between&& between) {
  constexpr int NMT = VHSP / 32;
  static_assert(NMT == 16, "four waves x four 32-channel blocks x four row blocks");
  constexpr int VSTEPS = 32;
  const uint32_t plane = (uint32_t)(threadIdx.x & 63) * 16u;

  // The registers an LDS read (inline assembly) writes are filled when the
  // read completes, so nothing may copy them before the lgkmcnt wait that
  // covers the read: fragments used by several MFMAs are waited for in place
  // (vf/p0/p1 are the read destinations themselves; the two transposing reads
  // of a V^T fragment land in the halves of one register tuple), and a
  // fragment is never rebuilt by VALU moves right before the MFMA that reads
  // it (an inline-assembly MFMA gets no hazard wait states from the compiler).
  // V^T fragment (ks, c): 32 channels x 16 keys of this wave's channel block c.
  u32x4_t vf[4], p0[4], p1[4];
  auto v_frag = [&](auto KS, auto C) {
    constexpr int ks = decltype(KS)::value, c = decltype(C)::value;
    constexpr int off = ks * 16 * MlaLds<HSP>::ROWB + (c >> 1) * 128;
    const u32x2_t r0 = ds_read_tr16_b64_asm<off>(Lv + vaddr[c & 1]);
    const u32x2_t r1 = ds_read_tr16_b64_asm<off>(Lv + vaddr[2 + (c & 1)]);
    vf[c] = u32x4_t{r0[0], r0[1], r1[0], r1[1]};
  };
  auto p_frag = [&](auto KS, auto R) -> u32x4_t {
    constexpr int ks = decltype(KS)::value, r = decltype(R)::value;
    return ds_read_b128_asm<(2 * r + ks) * 1024>(Lp + plane);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  static_for<0, 4>([&](auto R) { p0[decltype(R)::value] = p_frag(I0{}, R); });
  v_frag(I0{}, I0{});
  v_frag(I0{}, I1{});
  static_for<0, VSTEPS>([&](auto N) {
    constexpr int n = decltype(N)::value;
    constexpr int ks = n / 16, c = (n / 4) % 4, r = n % 4;
    u32x4_t& b = ks == 0 ? p0[r] : p1[r];
    // Wait where a fragment is first used: V^T(ks, c) at r == 0, P(ks, r)
    // at c == 0 (later uses find it complete).
    if constexpr (r == 0 || c == 0) lgkm_wait_fence<PvSched::wait(n)>();
    PvMfma<DT>::run(st.o[4 * c + r], vf[c], b);
    // Reads issued after this MFMA (PvSched::at).
    if constexpr (n == 0) v_frag(I0{}, std::integral_constant<int, 2>{});
    if constexpr (n == 4) v_frag(I0{}, std::integral_constant<int, 3>{});
    if constexpr (n == 8) {
      v_frag(I1{}, I0{});
      p1[0] = p_frag(I1{}, I0{});
      p1[1] = p_frag(I1{}, I1{});
    }
    if constexpr (n == 10) {
      p1[2] = p_frag(I1{}, std::integral_constant<int, 2>{});
      p1[3] = p_frag(I1{}, std::integral_constant<int, 3>{});
    }
    if constexpr (n == 12) v_frag(I1{}, I1{});
    if constexpr (n == 16) v_frag(I1{}, std::integral_constant<int, 2>{});
    if constexpr (n == 20) v_frag(I1{}, std::integral_constant<int, 3>{});
    between(N);
    __builtin_amdgcn_sched_barrier(0);
  });
}

// NT: the tile copies take the streaming cache policy (launched for
// decode-shaped calls, where no other query tile re-reads a KV row).
template <typename DT, int HSP, int VHSP, bool NT>
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
  constexpr int PB_BYTES = 2 * NW * 2 * 1024;   // two P buffers: [2][row block][k-step][64 lanes x 16 B]
  constexpr int LDS_BYTES = NB * BUF_BYTES + PB_BYTES;
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

  const int wr = range_of_block(p.header);
  int u = ld_uniform(p.wg_range + wr);
  const int u_end = ld_uniform(p.wg_range + wr + 1);
  if (u >= u_end) return;
  int i = ld_uniform(p.wg_tile + wr);   // query tile holding unit u
  const int i_first = i;
  const bool softcap_on = p.softcap > 0.0f;

  // Copy slot sl = it * 64 + lane of this wave is LDS row 8 w + sl / CPR,
  // position sl % CPR, which holds chunk (sl % CPR) ^ swizzle(row). Its source
  // is byte load_off[it] of the wave's KW cache rows (one register per copy
  // instruction, so a copy needs no offset arithmetic). Chunks at channels
  // >= hs get 0xFFFF, past the descriptor's range.
  uint32_t load_off[LOADS];
#pragma unroll
  for (int it = 0; it < LOADS; ++it) {
    const int sl = it * 64 + lane;
    const int k = sl / CPR;
    const int lc = (sl - k * CPR) ^ mla_swizzle(w * KW + k);
    load_off[it] = lc * 8 < p.hs ? (uint32_t)((k * p.hs + lc * 8) * 2) : 0xFFFFu;
  }

  const int n_tiles = ld_uniform(p.header + 1);   // query tiles of the schedule
  while (u < u_end && i < n_tiles) {
    const MTile t = ld_uniform_tile(p.mt + i);
    const int next0 = ld_uniform(&p.mt[i + 1].unit0);
    const int ua = u;
    const int ub = min(u_end, next0);
    const int tile_a = t.kv_lo / KT + (ua - t.unit0);
    const int tile_b = tile_a + (ub - ua);
    const bool whole = (ua == t.unit0) && (ub == next0);
    const int b = t.b;
    const int cum_b = t.tok0;
    const int past_b = t.past;

    // This lane's query row (rows past the tile read row 0 of the tile and are
    // never stored; each row's softmax and output column are independent).
    const int rloc = w * 32 + (fresh_lane() & 31);   // re-derived per piece: nothing lane-derived is kept in a spill slot
    const bool row_ok = rloc < t.nrows;
    const int R = t.row0 + (row_ok ? rloc : 0);
    const int tq = R / p.H;
    const int h = R - tq * p.H;
    const int pos = past_b + tq;
    const int lo_row = p.window >= 0 ? max(0, pos - p.window) : 0;
    const int64_t qrow = (int64_t)(cum_b + tq) * p.H + h;
    // Wave-uniform visibility bounds over the wave's valid rows: a tile with
    // lo_max <= first key and last key <= pos_min needs no masking. The valid
    // rows are consecutive and both pos and lo_row grow with the row, so the
    // bounds are those of the wave's first and last valid row (scalar work;
    // a cross-lane reduction here costs permute addresses that the compiler
    // keeps in spill slots).
    int pos_min = INT_MAX, lo_max = INT_MIN;
    {
      const int nval = min(32, t.nrows - 32 * w);
      if (nval > 0) {
        const int r0 = t.row0 + 32 * w;
        pos_min = past_b + r0 / p.H;
        const int pos1 = past_b + (r0 + nval - 1) / p.H;
        lo_max = p.window >= 0 ? max(0, pos1 - p.window) : 0;
      }
      pos_min = __builtin_amdgcn_readfirstlane(pos_min);
      lo_max = __builtin_amdgcn_readfirstlane(lo_max);
    }
    auto tile_full = [&](int key0) { return key0 >= lo_max && key0 + KT - 1 <= pos_min; };

    // Copy KV tile `tile` into LDS buffer `bufi`: exactly LOADS copy
    // instructions per wave (vmcnt counts them).
    // Block id of the cache block holding this wave's keys of `tile`.
    auto block_of = [&](int tile) -> int {
      const int kw0 = tile * KT + w * KW;
      return ld_uniform(p.bt + (int64_t)b * p.MB + min(kw0 >> p.bs_log2, p.MB - 1));
    };
    // A planned tile copy: descriptor over the wave's KW cache rows, LDS
    // destination. Keys at or past kv_hi (and every key of a tile past the
    // piece) lie past the descriptor's range and land as zeros, so the only
    // per-lane masking left is for keys below kv_lo (`lower`, rare: the first
    // tile of a piece whose range does not start on a tile boundary).
    struct CopyPlan {
      u32x4_t rsrc;
      uint32_t dst0;
      int kw0;
      bool lower;
    };
    auto plan = [&](int tile, int bufi, int blk_raw) -> CopyPlan {
      CopyPlan c;
      c.kw0 = tile * KT + w * KW;
      const int blk = clamp_block(blk_raw, p.nblk);
      const uint16_t* rows = p.cache + (((int64_t)blk << p.bs_log2) + (c.kw0 & ((1 << p.bs_log2) - 1))) * p.hs;
      const int nkeys = tile < tile_b ? min(max(t.kv_hi - c.kw0, 0), KW) : 0;
      c.rsrc = rsrc_words_u(rows, (uint32_t)(nkeys * p.hs * 2));
      c.dst0 = lds_addr(lds_raw) + (uint32_t)(bufi * BUF_BYTES + w * SLOTS * 16);
      c.lower = tile < tile_b && c.kw0 < t.kv_lo;
      return c;
    };
    // Copy instruction `it` of a planned tile (LDS slots it*64 .. it*64+63 of
    // the wave's slice). Exactly LOADS of them per tile and wave (vmcnt counts
    // them). LOWER: keys below kv_lo take an out-of-range offset.
    auto copy_one = [&](const CopyPlan& c, int it, auto LOWER) {
      uint32_t off = load_off[it];
      if constexpr (decltype(LOWER)::value) {
        const int j = c.kw0 + (it * 64 + opaque_lane()) / CPR;
        off = j >= t.kv_lo ? off : kOutOfRange;
      }
      copy16_to_lds<NT>(c.dst0 + it * 64 * 16, off, c.rsrc);
    };
    auto issue = [&](int tile, int bufi, int blk_raw) {
      const CopyPlan c = plan(tile, bufi, blk_raw);
      if (c.lower) {
#pragma unroll
        for (int it = 0; it < LOADS; ++it) copy_one(c, it, std::true_type{});
      } else {
#pragma unroll
        for (int it = 0; it < LOADS; ++it) copy_one(c, it, std::false_type{});
      }
    };

    // Tiles tile_a and tile_a + 1 of the first pass go out before the query.
#pragma unroll
    for (int k = 0; k < NB - 2; ++k) issue(tile_a + k, k, block_of(min(tile_a + k, tile_b - 1)));

    // Query fragments (k-step s holds channels 16 s + 8 hi .. + 8 of the row),
    // from the copy the schedule launch wrote in fragment
    // order with RoPE applied (qfrag): the wave's 32-row block (nv rows) holds
    // 8-channel chunk c of its row l at chunk c * nv + l, so k-step s of lane
    // (l, hi) is chunk (2 s + hi) nv + l and every load reads one contiguous
    // run. A wave with no row of the tile reads the tile's first block; lanes
    // past their block's rows read its row 0 (they never vote or store). One
    // descriptor covers exactly the block read.
    MlaState<HSP, VHSP> st;
    const int64_t trow0 = (int64_t)cum_b * p.H + t.row0;   // first query row of the tile
    {
      const int nvw = min(32, t.nrows - 32 * w);            // the wave's own rows
      const int nvb = nvw > 0 ? nvw : min(32, t.nrows);     // rows of the block read
      const int64_t brow = trow0 + (nvw > 0 ? 32 * w : 0);  // its first row
      const u32x4_t qrs = rsrc_words_u(p.qfrag + brow * HSP, (uint32_t)(nvb * HSP * 2));
      const int ln = opaque_lane();
      const int l = (ln & 31) < nvb ? (ln & 31) : 0;
      const uint32_t lb = (uint32_t)((((ln >> 5) * nvb) + l) * 16);
#pragma unroll
      for (int s = 0; s < NKS; ++s) st.qf[s] = buffer_load_b128(qrs, lb + (uint32_t)(s * 32 * nvb));
    }

    // The first two KV tiles of the piece are already in flight (issued
    // before the query loads so that the two latencies overlap); the query
    // and they have landed before the tile loop starts (the compiler's own
    // wait for the query loads would otherwise sit inside the tile loop and
    // drain the copy pipeline on every tile): vmcnt(0), expcnt/lgkmcnt
    // unconstrained.
    __builtin_amdgcn_s_waitcnt(0x0F70);

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
      // This wave's value channels start at chunk 16 w (byte 256 w of the row;
      // the swizzle only permutes chunks within aligned groups of 8).
      for (int par = 0; par < 2; ++par) {
        vaddr[par] = k0b * CPR * 16 + (((4 * par + lcb) ^ sw0) << 4) + (cq & 1) * 8 + 256 * w;
        vaddr[2 + par] = (k0b + 8) * CPR * 16 + (((4 * par + lcb) ^ sw1) << 4) + (cq & 1) * 8 + 256 * w;
      }
    }
    const uint32_t lds0 = lds_addr(lds_raw);
    // P buffer of tile k: pbuf0 + ((k - tile_a) & 1) * (PB_BYTES / 2).
    const uint32_t pbuf0 = lds0 + NB * BUF_BYTES;

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
      // Every iteration issues the copies of one tile (empty past the piece),
      // so the copy wait below is the same on every tile. The first pass's
      // first AHEAD tiles were issued before the query loads.
      if (pass > 0) {
#pragma unroll
        for (int k = 0; k < AHEAD; ++k) issue(tile_a + k, k, block_of(min(tile_a + k, tile_b - 1)));
      }
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
      auto qk_step = [&](int tt, auto&& between) -> f32x16_t {
        static_assert(AHEAD == 2, "one tile of copies in flight beyond tile tt");
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS) : "memory");
        lds_barrier();   // tile tt complete; every wave is done with tile tt - 2
        // Copies of tile tt + AHEAD go out during the QK MFMAs of tile tt; their
        // block id was read one iteration earlier.
        const int blk_cur = blk_next;
        blk_next = block_of(min(tt + AHEAD + 1, tile_b - 1));
        const CopyPlan cp = plan(tt + AHEAD, (uint32_t)(tt + AHEAD - tile_a) & (NB - 1), blk_cur);
        const uint32_t L = lds0 + ((uint32_t)(tt - tile_a) & (NB - 1)) * BUF_BYTES;
        if (cp.lower)
          return mla_qk<DT, HSP, LOADS>(
              st.qf, L, kaddr, [&](auto IT) { copy_one(cp, decltype(IT)::value, std::true_type{}); }, between);
        return mla_qk<DT, HSP, LOADS>(
            st.qf, L, kaddr, [&](auto IT) { copy_one(cp, decltype(IT)::value, std::false_type{}); }, between);
      };
      // Iteration tt: QK(tt), then PV(tt - 1) with the softmax of tt between
      // its MFMAs (step c after PV MFMA 2 c + 1); P(tt) goes to the P buffer
      // of tt's parity. PV(tt - 1) reads P(tt - 1), which every wave wrote
      // before this iteration's first barrier; the buffer P(tt) overwrites
      // was last read by PV(tt - 2), before that barrier too.
      auto tile_lds = [&](int tt) -> uint32_t { return lds0 + ((uint32_t)(tt - tile_a) & (NB - 1)) * BUF_BYTES; };
      auto pbuf = [&](int tt) -> uint32_t { return pbuf0 + ((uint32_t)(tt - tile_a) & 1) * (PB_BYTES / 2); };
      auto noop = [](auto) {};
      {
        MlaSm sm;
        sm.s = qk_step(tile_a, noop);
        static_for<0, kSmChunks>([&](auto C) {
          mla_sm_chunk<DT, HSP, VHSP, decltype(C)::value>(st, sm, tile_a * KT, rpos, lo_row, tile_full(tile_a * KT),
                                                          softcap_on, p);
        });
        mla_sm_store(sm, pbuf(tile_a));
      }
      for (int tt = tile_a + 1; tt < tile_b; ++tt) {
        MlaSm sm;
        sm.s = qk_step(tt, noop);
        const int key0 = tt * KT;
        const bool full = tile_full(key0);
        mla_pv<DT, HSP, VHSP>(st, tile_lds(tt - 1), vaddr, pbuf(tt - 1), [&](auto N) {
          constexpr int n = decltype(N)::value;
          if constexpr (n % 2 == 1 && n / 2 < kSmChunks)
            mla_sm_chunk<DT, HSP, VHSP, n / 2>(st, sm, key0, rpos, lo_row, full, softcap_on, p);
        });
        mla_sm_store(sm, pbuf(tt));
      }
      // PV of the last tile (its buffer is still resident) once every wave's
      // P of that tile is in LDS.
      lds_barrier();
      mla_pv<DT, HSP, VHSP>(st, tile_lds(tile_b - 1), vaddr, pbuf(tile_b - 1), noop);
      // The last copies (tiles past the piece, zero-filled) land before the
      // tile buffers are reused below.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      // Whole-workgroup vote on a second pass (the tile buffers are free once
      // every wave passed the barrier; the flags sit in the first buffer).
      lds_barrier();
      int* const vote = (int*)lds_raw;
      // Every lane takes part in the ballot (taken before the one-lane
      // store); rows past the tile (duplicates of its row 0, unmasked where
      // the wave has no valid row) do not vote.
      const int vl = fresh_lane();
      const bool any_ovf = __any(st.ovf && (w * 32 + (vl & 31) < t.nrows));
      if (vl == 0) vote[w] = any_ovf ? 1 : 0;
      lds_barrier();
      const int again = vote[0] | vote[1] | vote[2] | vote[3];
      lds_barrier();     // votes read before the buffers are reused
      if (!again) break;
      st.m_ref = st.m_seen;
    }
    // PV accumulators are read below (LDS writes from AGPRs).
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

    // Epilogue through LDS (the tile buffers are free): O^T of all rows is
    // staged as float32 rows in two rounds, round k holding channel blocks
    // 2k, 2k + 1 of every wave (wave w's 64 channels at staged column 64 w),
    // written straight from the accumulation registers; then every thread
    // normalises 8 consecutive channels of a row and stores them, rounded to
    // the output type, with coalesced stores into the output (whole tile) or
    // the piece's partial slot (split-KV; (m, l) go beside it in float32).
    // Rows are padded by 16 bytes against bank conflicts.
    const float l_tot = sum_xor32(st.l_run);
    constexpr int QCH = VHSP / NW;                         // value channels per wave
    constexpr int RCH = QCH / 2;                           // per wave and round
    constexpr int SCOL = NW * RCH;                         // staged columns per round
    constexpr int ORS = SCOL + 4;                          // floats per staged row
    constexpr int C8 = SCOL / 8;                           // 8-channel groups per staged row
    static_assert((RW * ORS + 2 * RW) * 4 <= NB * BUF_BYTES, "epilogue staging fits the tile buffers");
    static_assert(RCH == 64, "two 32-channel blocks per wave and round");
    float* const ost = (float*)lds_raw;
    float* const rowl = ost + RW * ORS;                    // [RW] denominators
    // Lane quantities re-derived here rather than carried across the tile loop.
    const int eln = fresh_lane();
    const int el32 = eln & 31, ehi = eln >> 5;
    const int erloc = w * 32 + el32;
    const int etid = w * 64 + eln;
    if (ehi == 0) rowl[erloc] = l_tot;
    // Partial slot of a split piece: the workgroup's first piece goes to slot
    // wr, a later one to G + tile.
    const int64_t slot = whole ? 0 : (i == i_first ? (int64_t)wr : (int64_t)gridDim.x + i);
    if (!whole && ehi == 0 && erloc < t.nrows) {
      float* ml = p.part_ml + (slot * RW + erloc) * 2;
      ml[0] = st.m_ref;
      ml[1] = l_tot;
    }
    // Lane's staging address for row block r: row 32 r + l32, column 64 w + 4 hi.
    uint32_t wb[NW];
#pragma unroll
    for (int r = 0; r < NW; ++r) wb[r] = lds_addr(ost) + (uint32_t)(((32 * r + el32) * ORS + RCH * w + 4 * ehi) * 4);
    const int64_t orow0 = (int64_t)cum_b * p.H + t.row0;  // output row of local row 0
    // Read-out of a full tile (every row, every value channel): RSTEP rows per
    // pass of the workgroup, NIT passes, reciprocals of the rows' denominators
    // formed once for both rounds.
    const bool full_tile = t.nrows == RW && p.vhs == VHSP;
    constexpr int RSTEP = NW * 64 / C8;
    constexpr int NIT = RW / RSTEP;
    constexpr int NBT = 4;
    static_assert(NIT % NBT == 0, "whole batches");
    const int r0f = etid / C8;
    // (Defined on every path: an undefined array would let the compiler carry
    // the previous piece's values around the piece loop.)
    float inv_r[NIT];
#pragma unroll
    for (int k = 0; k < NIT; ++k) inv_r[k] = 0.0f;
    static_for<0, 2>([&](auto RD) {
      constexpr int rd = decltype(RD)::value;
      static_for<0, 2 * NW * 4>([&](auto K) {
        constexpr int kk = decltype(K)::value;
        constexpr int cl = kk / (NW * 4), r = (kk / 4) % NW, j = kk % 4;
        constexpr int c = 2 * rd + cl;
        const f32x4_t part = __builtin_shufflevector(st.o[4 * c + r], st.o[4 * c + r], 4 * j, 4 * j + 1, 4 * j + 2,
                                                     4 * j + 3);
        ds_write_b128_acc<(32 * cl + 8 * j) * 4>(wb[r], part);
      });
      lds_barrier();     // staged round visible (the asm writes are waited for by lgkmcnt(0))
      if (full_tile) {
        // Every row and channel present: thread (r0, c8) handles staged column
        // group c8 of rows r0, r0 + RSTEP, ...: the staging reads of a batch
        // of NBT rows go out before its stores, with no per-item tests (with
        // one wave per SIMD nothing else hides an LDS round trip per row).
        const int c8 = etid % C8;
        const int sc = c8 * 8;
        const int cg = (sc / RCH) * QCH + rd * RCH + (sc % RCH);
        if constexpr (rd == 0) {
#pragma unroll
          for (int k = 0; k < NIT; ++k) {
            const float lr = rowl[r0f + RSTEP * k];
            inv_r[k] = lr > 0.0f ? 1.0f / lr : 0.0f;
          }
        }
        // Element offsets of row r0f: output (whole tile) or partial slot.
        const int64_t dst0 = whole ? (orow0 + r0f) * VHSP + cg : slot * p.part_slot + (int64_t)r0f * p.part_row + cg;
        const int64_t dstep = whole ? (int64_t)RSTEP * VHSP : (int64_t)RSTEP * p.part_row;
        const float* const src0 = ost + r0f * ORS + sc;
#pragma unroll
        for (int k0 = 0; k0 < NIT; k0 += NBT) {
          f32x4_t v0[NBT], v1[NBT];
#pragma unroll
          for (int k = 0; k < NBT; ++k) {
            v0[k] = *(const f32x4_t*)(src0 + (k0 + k) * RSTEP * ORS);
            v1[k] = *(const f32x4_t*)(src0 + (k0 + k) * RSTEP * ORS + 4);
          }
#pragma unroll
          for (int k = 0; k < NBT; ++k) {
            const float inv = inv_r[k0 + k];
            const float x[8] = {v0[k][0] * inv, v0[k][1] * inv, v0[k][2] * inv, v0[k][3] * inv,
                                v1[k][0] * inv, v1[k][1] * inv, v1[k][2] * inv, v1[k][3] * inv};
            if (whole) *(u32x4_t*)(p.out + dst0 + (k0 + k) * dstep) = pack8<DT>(x);
            else store_part8<DT>(p.part_o, dst0 + (k0 + k) * dstep, x);
          }
        }
      } else for (int idx = etid; idx < RW * C8; idx += NW * 64) {
        const int r = idx / C8;
        const int sc = (idx - r * C8) * 8;                 // staged column
        const int cg = (sc / RCH) * QCH + rd * RCH + (sc % RCH);   // value channel
        if (r >= t.nrows || cg >= p.vhs) continue;
        const f32x4_t v0 = *(const f32x4_t*)(ost + r * ORS + sc);
        const f32x4_t v1 = *(const f32x4_t*)(ost + r * ORS + sc + 4);
        const float lr = rowl[r];
        const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
        const float x[8] = {v0[0] * inv, v0[1] * inv, v0[2] * inv, v0[3] * inv,
                            v1[0] * inv, v1[1] * inv, v1[2] * inv, v1[3] * inv};
        // Output row, or the piece's partial row (padded to VHSP channels).
        if (!whole) {
          store_part8<DT>(p.part_o, slot * p.part_slot + (int64_t)r * p.part_row + cg, x);
        } else {
          uint16_t* dst = p.out + (orow0 + r) * p.vhs + cg;
          if (cg + 8 <= p.vhs && (p.vhs & 7) == 0) {
            *(u32x4_t*)dst = pack8<DT>(x);
          } else {
            for (int k = 0; k < 8 && cg + k < p.vhs; ++k) dst[k] = (uint16_t)DT::from_f32(x[k]);
          }
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
  hipError_t PA_ATTN_FN(lat, DTN, HSP, VHSP, 4, 32, occ)(int* n) {                                           \
    void (*fn)(AttnParams) = attn_mla_kernel<DT, HSP, VHSP, true>;                                      \
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, reinterpret_cast<const void*>(fn), 256, 0);  \
  }                                                                                                     \
  hipError_t PA_ATTN_FN(lat, DTN, HSP, VHSP, 4, 32, launch)(const AttnParams& p, int grid, bool combine,      \
                                                       int cgrid, hipStream_t s, const hipEvent_t* ev) { \
    hipError_t e = ev ? hipEventRecord(ev[0], s) : hipSuccess;                                          \
    if (e != hipSuccess) return e;                                                                      \
    if (p.kv_stream) attn_mla_kernel<DT, HSP, VHSP, true><<<grid, 256, 0, s>>>(p);                      \
    else attn_mla_kernel<DT, HSP, VHSP, false><<<grid, 256, 0, s>>>(p);                                 \
    e = hipGetLastError();                                                                              \
    if (e == hipSuccess && ev) e = hipEventRecord(ev[1], s);                                            \
    if (e != hipSuccess || !combine) return e;                                                          \
    combine_kernel<DT, VHSP, 128><<<dim3(cgrid, 128 / CombineShape<VHSP>::ROWS), 256, 0, s>>>(p);        \
    return hipGetLastError();                                                                           \
  }                                                                                                     \
  }
