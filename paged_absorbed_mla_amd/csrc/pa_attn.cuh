// Read phase of paged LATENT attention on gfx950: MFMA attention over LDS-staged
// paged latent tiles, and the split-KV combine.
//
// Semantics: docs.rs page "onnx-runtime-ep-cuda src/kernels/paged_attention.rs",
// "LATENT semantics" (read phase) and device function attn_impl: per (token,
// head), partial RoPE of the query, causal keys j <= pos with pos - j <= window
// when a window is set, scale then softcap, online softmax with
// corr = exp(m_old - m_new) (0 when m_old = -inf), V = leading v_head_size
// channels of the same cached row, output acc / denom (0 when denom = 0).
//
// Design (not the page's: its kernel runs one 128-thread block per (token,
// head), re-reads the whole context per head and reduces each dot product
// with a shared-memory tree):
//   * A workgroup owns a query tile of 32 * NW rows of one sequence (row =
//     token_in_sequence * H + head, so consecutive rows are consecutive in
//     `query` and `output`) and walks a contiguous range of KV tiles of KT keys.
//   * Each KV tile (KT latent rows x HSP channels) is copied from the paged
//     cache into LDS once, with direct global->LDS loads (no VGPR staging),
//     double buffered, and shared by every row of the workgroup: QK^T reads all
//     HSP channels and PV reads the first VHSP channels of the same LDS rows.
//   * QK^T is computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16: A = 32
//     keys x 16 channels from LDS (one 16-byte read per lane), B = the wave's
//     32 query rows, kept in registers after RoPE. The accumulator then holds
//     one query row per lane (two lanes per row), so the softmax running max
//     and sum live in that lane's registers and need a single cross-lane max.
//   * PV is computed transposed too, O^T = V^T P^T: B = P^T comes straight from
//     the S^T accumulator registers (the key order inside a 16-key step is
//     permuted consistently on both operands), A = V^T is read from the
//     key-major LDS tile with ds_read_b64_tr_b16 transposing loads. O^T keeps
//     one query row per lane as well, so rescaling by the running-max
//     correction is a per-lane multiply.
//   * LDS rows are XOR-swizzled per 16-byte chunk (low three bits of the chunk
//     index ^= (key & 7) ^ (key >> 3 & 1)) against bank conflicts on the
//     column-wise reads; the global->LDS copy applies the same swizzle on the
//     global side, so every copy instruction still writes 1 KB contiguously.
//   * Keys outside the query tile's range are loaded from a zero page, so a
//     masked probability (0) never meets a non-finite cache value.
//   * Work split (flash-decoding): an on-device scheduler lays the KV tiles of
//     all query tiles end to end and gives every workgroup an equal share.
//     A query tile whose tiles span several workgroups gets one partial per
//     piece (float32 max and denominator, normalised output: bfloat16 for
//     bfloat16 outputs, float32 for float16 ones), merged by the combine
//     kernel with a log-sum-exp weighting.
#pragma once

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// One query tile: rows [row0, row0 + nrows) of sequence b. A row is
// token * H + head within the sequence, H the query heads that share one
// key/value head (all of them in the latent layout). In the separate
// (grouped-query) layout each sequence is scheduled once per key/value head
// kvg, whose query heads are kvg * H .. kvg * H + H - 1.
struct MTile {
  int32_t b, row0, nrows, kv_lo, kv_hi;
  int32_t unit0;      // first global work unit (one unit = one KV tile)
  int32_t part_base;  // first partial slot, -1 when one workgroup covers the tile
  int32_t w_first;    // workgroup that processes the tile's first unit
  int32_t npieces;    // workgroups that process the tile
  int32_t tok0;       // first token of sequence b (cumulative_sequence_length, clamped into [0, T])
  int32_t past;       // past length of sequence b (clamped into [0, max_blocks_per_seq * block_size])
  int32_t kvg;        // key/value head of the tile (0 in the latent layout)
};
static_assert(sizeof(MTile) == 48, "MTile layout");

struct AttnParams {
  const uint16_t* query;
  const uint16_t* cache;
  const uint16_t* cos_t;
  const uint16_t* sin_t;
  const int32_t* bt;
  uint16_t* out;
  const int32_t* header;    // [0] work units U, [1] query tiles M, [2] unit ranges in use
  const int32_t* wg_range;  // [grid + 1] unit range of each workgroup
  const int32_t* wg_tile;   // [grid] query tile holding each workgroup's first unit
  const MTile* mt;          // [M + 1], mt[M].unit0 = U
  float* part_ml;           // [slots][rows][2]: running max (log2 domain), denominator
  void* part_o;             // partial outputs acc / l (element type PartT<DT>): slot s, row r at s * part_slot + r * part_row
  int64_t part_slot;        // elements between slots (padded: not a power of two)
  int part_row;             // elements between rows (VHSP + 16 bytes)
  const uint16_t* qfrag;    // [T * H][HSP]: RoPE'd query in fragment order (four-wave 576 kernel)
  const uint16_t* vcache;   // separate layout: value cache [slots][kvh][vhs] (null in the latent layout)
  int nblk;                 // num_blocks (< 2^31 / block_size): block ids are clamped into [0, nblk)
  int kv_stream;            // 1: every KV row is read by one query tile only (a decode-shaped call)
  int many_pieces;          // 1: split-KV leaves many pieces per query tile (see CombineShape)
  int64_t prow;             // rotary table rows: positions are clamped into [0, prow)
  int H;                    // query heads per key/value head (rows per token of a query tile)
  int Hq;                   // query heads of the call (H * kvh): head stride of query and output rows
  int krs, vrs;             // elements between cache slots: key cache (kvh * hs), value cache (kvh * vhs)
  int hs, vhs, bs_log2, MB;
  int ro, rd, do_rotary, interleaved, window;
  float scale, scale_log2, softcap, softcap_inv;
};

constexpr float kLog2e = 1.4426950408889634f;

// Build-time tunables of the generic kernel (defaults measured best; other
// values for A/B timing): fragment prefetch depths of the tile computation
// (K fragments for QK, V^T fragments for PV) and LDS tile buffers (one-wave
// instances, four-wave instances) where two workgroups still fit in a CU.
#ifndef PA_GEN_QPF
#define PA_GEN_QPF 4
#endif
#ifndef PA_GEN_VPF
#define PA_GEN_VPF 3
#endif
#ifndef PA_GEN_NBUF
#define PA_GEN_NBUF 3
#endif
#ifndef PA_GEN_NBUF4
#define PA_GEN_NBUF4 3
#endif
// Wave priority: 1 raises it for the MFMA phases of a tile (QK, PV) and drops
// it for the softmax, so that of the two workgroups sharing a CU the one with
// matrix work issues first and the other's vector work fills the gaps between
// its MFMAs; 0 alternates it every tile instead (four-wave instances).
#ifndef PA_GEN_PRIO
#define PA_GEN_PRIO 1
#endif
// Split-KV combine shape: threads per row (at most), pieces per memory round trip.
#ifndef PA_COMB_TPR
#define PA_COMB_TPR 64
#endif
#ifndef PA_COMB_QA
#define PA_COMB_QA 4
#endif

// Element type of the split-KV partial outputs. bfloat16 outputs keep them in
// bfloat16: a second rounding (half an ulp, 2^-8 relative at most) stays well
// inside that type's output tolerance. float16 outputs keep them in float32:
// the float16 tolerance is about one rounding of an output near 4, with no
// room for a second.
template <typename DT> struct PartF32 : std::false_type {};
template <> struct PartF32<F16> : std::true_type {};

// Eight normalised channels of a row into a partial slot.
template <typename DT>
__device__ __forceinline__ void store_part8(void* part, int64_t off, const float (&x)[8]) {
  if constexpr (PartF32<DT>::value) {
    float* d = (float*)part + off;
    *(f32x4_t*)d = f32x4_t{x[0], x[1], x[2], x[3]};
    *(f32x4_t*)(d + 4) = f32x4_t{x[4], x[5], x[6], x[7]};
  } else {
    *(u32x4_t*)((uint16_t*)part + off) = pack8<DT>(x);
  }
}

// Eight channels of a partial slot, widened to float32.
template <typename DT>
__device__ __forceinline__ void load_part8(const void* part, int64_t off, float (&x)[8]) {
  if constexpr (PartF32<DT>::value) {
    const f32x4_t a = *(const f32x4_t*)((const float*)part + off);
    const f32x4_t b = *(const f32x4_t*)((const float*)part + off + 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) { x[k] = a[k]; x[4 + k] = b[k]; }
  } else {
    unpack8<DT>(*(const u32x4_t*)((const uint16_t*)part + off), x);
  }
}

// Chunk swizzle of LDS row `key`: period 16 in the key, so rows 16 apart share
// it and their addresses differ by a compile-time constant. Rows k and k + 8
// differ in the low bit; within any aligned 8 (or 16) rows the values are
// distinct (combined with the row parity for 16).
__device__ __forceinline__ int lds_swizzle(int key) { return (key & 7) ^ ((key >> 3) & 1); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 32-bit LDS address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// ds_read_b64_tr_b16 at LDS address addr + OFF, issued without compiler
// dependency tracking: the caller waits (lgkm_wait_n) before using the result.
template <int OFF>
__device__ __forceinline__ u32x2_t ds_read_tr16_b64_asm(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset is 16 bits");
  u32x2_t d;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "n"(OFF));
  return d;
}

// ds_read_b128 at LDS address addr + OFF, issued like ds_read_tr16_b64_asm.
template <int OFF>
__device__ __forceinline__ u32x4_t ds_read_b128_asm(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset is 16 bits");
  u32x4_t d;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(d) : "v"(addr), "n"(OFF));
  return d;
}

// The lane index, opaque to the optimiser: values derived from it are
// recomputed where they are used instead of being hoisted out of loops and
// kept live (and spilled) across them.
__device__ __forceinline__ int opaque_lane() {
  int l = (int)threadIdx.x & 63;
  asm volatile("" : "+v"(l));
  return l;
}

// Lane id formed afresh from the exec-mask bit count (no memory access): the
// opaque all-ones mask keeps the compiler from reusing an earlier lane id,
// which after a long loop would sit in a spill slot, and from holding values
// derived from it live across that loop.
__device__ __forceinline__ int fresh_lane() {
  uint32_t m = ~0u;
  asm volatile("" : "+s"(m));
  return (int)__builtin_amdgcn_mbcnt_hi(m, __builtin_amdgcn_mbcnt_lo(m, 0u));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Raw buffer descriptor over `bytes` bytes at `base` (stride 0, 32-bit data
// format word of the gfx9 descriptor layout). Loads at offsets >= bytes return
// zeros without touching memory.
constexpr uint32_t kOutOfRange = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One 16-byte-per-lane direct global->LDS copy: lane l's 16 bytes at buffer
// offset voff land at LDS address lds_base + 16 l. Issued as inline assembly
// so that the compiler does not see an LDS write it cannot order: it would
// otherwise drain every in-flight copy (vmcnt(0)) before the next LDS read.
// The caller orders copies against LDS reads with explicit vmcnt waits and a
// barrier. `rsrc` is a raw buffer descriptor (loads past its size read zeros).
// NT: non-temporal (streaming) cache policy, for data that no other
// workgroup reads again within the launch (a decode step's KV rows): such
// copies stream from HBM faster with it. Data that other query tiles re-read
// (prefill) keeps the default policy, which leaves it in L2 for them.
template <bool NT = false>
__device__ __forceinline__ void copy16_to_lds(uint32_t lds_base, uint32_t voff, u32x4_t rsrc) {
  // lds_base is wave-uniform by contract; readfirstlane keeps it in an SGPR
  // where the compiler cannot prove that (the "s" constraint needs one).
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(rsrc) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(rsrc) : "memory", "m0");
}

// Raw buffer descriptor words over `bytes` bytes at `base` (stride 0, the same
// descriptor make_rsrc builds).
__device__ __forceinline__ u32x4_t rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}

// rsrc_words for a wave-uniform base: the words are forced into SGPRs.
__device__ __forceinline__ u32x4_t rsrc_words_u(const void* base, uint32_t bytes) {
  u32x4_t r = rsrc_words(base, bytes);
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = __builtin_amdgcn_readfirstlane(r[k]);
  return r;
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// s_waitcnt vmcnt(ahead * PER) for a runtime ahead in [0, MAXA] (the count is an
// immediate, so each value gets its own instruction).
template <int PER, int MAXA>
__device__ __forceinline__ void vm_wait_tiles(int ahead) {
  if constexpr (MAXA >= 2) {
    if (ahead >= 2) { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER) : "memory"); return; }
  }
  if constexpr (MAXA >= 1) {
    if (ahead >= 1) { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER) : "memory"); return; }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Workgroup barrier that orders LDS only: the wave's own LDS operations
// complete (lgkmcnt(0)) before it arrives. __syncthreads() would also drain
// every outstanding global->LDS copy (its workgroup fence makes the compiler
// emit vmcnt(0)), which serialises a multi-buffer copy pipeline; here copies
// are awaited explicitly, per tile, with vmcnt before the barrier. The memory
// clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int N>
__device__ __forceinline__ void lgkm_wait_n() {
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}

// softcap * tanh(scale * s / softcap), returned in log2 units (times log2 e).
// tanh(z) = 1 - 2 / (e^{2z} + 1): saturates to +-1 for large |z| (e^{2z} = inf
// or 0) and has absolute error ~1e-7 near 0, i.e. ~softcap * 1e-7 on the score.
__device__ __forceinline__ float softcap_log2(float s, float scale, float cap, float cap_inv) {
  const float z = s * scale * cap_inv;
  const float e2z = fast_exp2(z * (2.0f * kLog2e));
  const float th = 1.0f - 2.0f * __builtin_amdgcn_rcpf(e2z + 1.0f);
  return cap * th * kLog2e;
}

// Scalar (s_load) read of data that no thread writes while the kernel runs:
// block_table, sequence lengths and the schedule the previous launch wrote.
__device__ __forceinline__ int ld_uniform(const int32_t* ptr) {
  return *(const __attribute__((address_space(4))) int32_t*)ptr;
}

// Unit range handled by this workgroup. Workgroups are dispatched to the
// eight XCDs (each with its own L2) round-robin by index, so when the grid is
// a multiple of eight, XCD x takes the consecutive ranges x * grid/8 ..
// (x + 1) * grid/8 - 1: ranges that share a query tile, and so read the same
// query rows, then mostly share an L2. When the schedule uses fewer ranges
// than workgroups (header[2], a short batch), range b goes to workgroup b,
// so the ranges in use spread over every XCD.
__device__ __forceinline__ int range_of_block(const int32_t* header) {
  const int g = (int)gridDim.x, b = (int)blockIdx.x;
  const int used = ld_uniform(header + 2);
  return ((g & 7) == 0 && used >= g) ? (b & 7) * (g >> 3) + (b >> 3) : b;
}

// Block id clamped into [0, nblk): a block_table entry outside the cache (a
// violated precondition) then reads some cache block instead of faulting.
__device__ __forceinline__ int clamp_block(int blk, int nblk) { return min(max(blk, 0), nblk - 1); }

__device__ __forceinline__ MTile ld_uniform_tile(const MTile* ptr) {
  const int32_t* q = (const int32_t*)ptr;
  MTile t;
  t.b = ld_uniform(q + 0);
  t.row0 = ld_uniform(q + 1);
  t.nrows = ld_uniform(q + 2);
  t.kv_lo = ld_uniform(q + 3);
  t.kv_hi = ld_uniform(q + 4);
  t.unit0 = ld_uniform(q + 5);
  t.part_base = ld_uniform(q + 6);
  t.w_first = ld_uniform(q + 7);
  t.npieces = ld_uniform(q + 8);
  t.tok0 = ld_uniform(q + 9);
  t.past = ld_uniform(q + 10);
  t.kvg = ld_uniform(q + 11);
  return t;
}

// Query / output row of row R (token * H + head) of a tile's sequence.
__device__ __forceinline__ int64_t head_row(const AttnParams& p, const MTile& t, int R) {
  const int tq = R / p.H;
  return (int64_t)(t.tok0 + tq) * p.Hq + t.kvg * p.H + (R - tq * p.H);
}

// State one wavefront carries across the KV tiles of a piece: its 32 query
// rows as MFMA B fragments, and the transposed output accumulators.
template <typename DT, int HSP, int VHSP, int KT, int QREG>
struct WaveState {
  static constexpr int NKR = QREG / 16;
  static constexpr int NMT = VHSP / 32;
  u32x4_t qf[NKR];
  f32x16_t o[NMT];
  float m_run, l_run;
};

// S^T = K Q^T for one LDS tile, softmax update, O^T += V^T P^T. K rows are
// at L (CPR chunks each), V rows at LV (VCPR chunks each; LV = L when V is
// the leading part of the latent row).
// after_qk() runs once the QK MFMAs are queued (the caller issues the second
// half of a later tile's copies there). GEN: the general score map (softcap,
// or a scale that is not positive); otherwise the raw scores go straight into
// the exponent (the common case, compiled without the other branches so that
// the scores stay in their registers).
template <typename DT, int HSP, int VHSP, int KT, int QREG, int VCPR, bool GEN, typename AfterQK>
__device__ __forceinline__ void tile_compute(WaveState<DT, HSP, VHSP, KT, QREG>& st, const uint8_t* L,
                                             const uint8_t* LV, const uint16_t* qrest, int key0, int pos,
                                             int lo_row, bool softcap_on, bool full, const AttnParams& p,
                                             AfterQK&& after_qk) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int CPR = HSP / 8;
  constexpr int NKK = HSP / 16;
  constexpr int NSUB = KT / 32;
  constexpr int NMT = VHSP / 32;
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Lane reads row l32 (+32 sub), chunk 2 kk + hi. Chunks 8 apart share the
  // swizzle, so four base addresses serve all kk with immediate offsets.
  const int swq = lds_swizzle(l32);
  const uint8_t* qb[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) qb[r] = L + l32 * CPR * 16 + (((2 * r + hi) ^ swq) << 4);
  // Software pipeline: the A fragment of step n is read QPF steps ahead; the
  // scheduling fences keep the compiler from hoisting all reads at once.
  // Channels [0, QREG) of the query come from registers, [QREG, HSP) from the
  // wave's persistent LDS rows (row l32, stride QRS elements).
  constexpr int NKR = QREG / 16;
  constexpr int QRS = HSP - QREG + 8;
  constexpr int QPF = PA_GEN_QPF;
  constexpr int QSTEPS = NSUB * NKK;
  f32x16_t s[NSUB];
#pragma unroll
  for (int sub = 0; sub < NSUB; ++sub) s[sub] = f32x16_t{};
  const uint16_t* qrow_lds = qrest + l32 * QRS + 8 * hi;
  auto qk_frag = [&](int n) -> u32x4_t {
    const int sub = n / NKK, kk = n % NKK;
    return *(const u32x4_t*)(qb[kk & 3] + sub * 32 * CPR * 16 + (kk >> 2) * 128);
  };
  auto q_frag = [&](int n) -> u32x4_t {
    const int kk = n % NKK;
    return *(const u32x4_t*)(qrow_lds + 16 * (kk - NKR));
  };
  if constexpr (PA_GEN_PRIO == 1) asm volatile("s_setprio 1");
  u32x4_t qa[QPF], qq[QPF];
#pragma unroll
  for (int n = 0; n < QPF; ++n) {
    qa[n] = qk_frag(n);
    if (n % NKK >= NKR) qq[n] = q_frag(n);
  }
#pragma unroll
  for (int n = 0; n < QSTEPS; ++n) {
    const u32x4_t cur = qa[n % QPF];
    const u32x4_t bq = (n % NKK < NKR) ? st.qf[(n % NKK) < NKR ? (n % NKK) : 0] : qq[n % QPF];
    if (n + QPF < QSTEPS) {
      qa[n % QPF] = qk_frag(n + QPF);
      if ((n + QPF) % NKK >= NKR) qq[n % QPF] = q_frag(n + QPF);
    }
    s[n / NKK] = DT::mfma32(cur, bq, s[n / NKK]);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (PA_GEN_PRIO == 1) asm volatile("s_setprio 0");
  after_qk();
  // Scores into log2 units, mask, tile max. Lane holds keys
  // hi*4 + (e&3) + 8*(e>>2) (+32 sub) of its row l32. With a positive scale
  // and no softcap the raw scores stay as they are: their max, times the
  // scale, is the max of the scaled scores (rounding is monotone), and the
  // scale is applied inside the exponent (one fma per score).
  if constexpr (GEN) {
    if (softcap_on) {
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[sub][e] = softcap_log2(s[sub][e], p.scale, p.softcap, p.softcap_inv);
    } else {
      const float sc = p.scale_log2;
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[sub][e] *= sc;   // element by element: a vector product would splat sc
    }
  }
  const float mul = GEN ? 1.0f : p.scale_log2;
  // `full` (wave-uniform): every row of the wave sees every key of the tile,
  // so no key is masked.
  if (!full) {
    // Key j = key0 + c of this lane's element is visible iff lo_row <= j <= pos,
    // i.e. c in [lo_row - key0, pos - key0] (c a compile-time constant).
    const int chi = pos - key0 - hi * 4, clo = lo_row - key0 - hi * 4;
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int c = sub * 32 + (e & 3) + 8 * (e >> 2);
        s[sub][e] = (c <= chi && c >= clo) ? s[sub][e] : -INFINITY;
      }
  }
  float tmax = -INFINITY;
#pragma unroll
  for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
    for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, s[sub][e]);
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * mul;   // -inf stays -inf (mul > 0)
  // Lazy rescale: the reference max moves only when the tile max exceeds it by
  // more than 8 (log2 units), so probabilities stay <= 2^8, and the O
  // accumulators are rescaled only when some row of the wave moved it. The
  // output is O / l with the same reference for both, so the result is exact.
  const bool bump = tmax > st.m_run + 8.0f;
  const float m_new = bump ? tmax : st.m_run;
  const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
  const float corr = fast_exp2(st.m_run - m_use);
  const bool rescale = bump && (st.m_run != -INFINITY);
  st.m_run = m_new;
  // The row sum adds the rounded probabilities (two per dot2 against (1, 1)),
  // the same values the PV product weights the rows with.
  u32x4_t pf[NSUB][2];
  float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // four partial sums: short dependency chains
#pragma unroll
  for (int sub = 0; sub < NSUB; ++sub) {
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(__builtin_fmaf(s[sub][8 * k2 + e], mul, -m_use));
      pf[sub][k2] = pack8<DT>(pv);
#pragma unroll
      for (int k = 0; k < 4; ++k) ps[k] = DT::sum2(pf[sub][k2][k], ps[k]);
    }
  }
  const float psum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
  st.l_run = st.l_run * corr + psum;
  if (__any(rescale)) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) st.o[mt][e] *= corr;
  }
  // O^T += V^T P^T. Transposing reads: lane (g, jj, cq) supplies key row jj and
  // channel quad cq of its 16-lane group; the group's lane i receives channel i
  // of the 4 keys.
  const int g = lane >> 4;
  const int jj = (lane & 15) >> 2;
  const int cq = lane & 3;
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  // Rows k0 = 16 step + (g >> 1) * 4 + jj and k1 = k0 + 8; the swizzle has
  // period 16, so two rows x two chunk parities give four base addresses.
  const int k0b = (g >> 1) * 4 + jj;
  const int sw0 = lds_swizzle(k0b), sw1 = lds_swizzle(k0b + 8);
  const int lcb = 2 * (g & 1) + (cq >> 1);
  const uint8_t* vb[2][2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    vb[0][par] = LV + k0b * VCPR * 16 + (((4 * par + lcb) ^ sw0) << 4) + (cq & 1) * 8;
    vb[1][par] = LV + (k0b + 8) * VCPR * 16 + (((4 * par + lcb) ^ sw1) << 4) + (cq & 1) * 8;
  }
  constexpr int VPF = PA_GEN_VPF;
  constexpr int VSTEPS = NSUB * 2 * NMT;
  auto pv_frag = [&](int n) -> u32x4_t {
    const int step = n / NMT, mt = n % NMT;        // step = sub * 2 + k2
    const int coff = step * 16 * VCPR * 16 + (mt >> 1) * 128;
    const i16x4_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb[0][mt & 1] + coff));
    const i16x4_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb[1][mt & 1] + coff));
    const u32x2_t d0 = __builtin_bit_cast(u32x2_t, r0);
    const u32x2_t d1 = __builtin_bit_cast(u32x2_t, r1);
    return u32x4_t{d0[0], d0[1], d1[0], d1[1]};
  };
  if constexpr (PA_GEN_PRIO == 1) asm volatile("s_setprio 1");
  u32x4_t va[VPF];
#pragma unroll
  for (int n = 0; n < VPF; ++n) va[n] = pv_frag(n);
#pragma unroll
  for (int n = 0; n < VSTEPS; ++n) {
    const u32x4_t cur = va[n % VPF];
    if (n + VPF < VSTEPS) va[n % VPF] = pv_frag(n + VPF);
    const int step = n / NMT;
    st.o[n % NMT] = DT::mfma32(cur, pf[step >> 1][step & 1], st.o[n % NMT]);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (PA_GEN_PRIO == 1) asm volatile("s_setprio 0");
#endif  // __HIP_DEVICE_COMPILE__
}

// SEP: separate (grouped-query) layout -- K rows from the key cache, V rows
// from the value cache into a second part of each LDS buffer; otherwise V is
// the leading VHSP channels of the latent row already in the buffer.
template <typename DT, int HSP, int VHSP, int NW, int KT, int QREG, bool SEP, bool GEN>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW >= 4 ? 2 : 1))) void attn_kernel(AttnParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int CPR = HSP / 8;          // 16-byte chunks per LDS row
  constexpr int VCPR = SEP ? VHSP / 8 : CPR;
  constexpr int TILE_CHUNKS = KT * CPR;
  constexpr int VTILE_CHUNKS = SEP ? KT * VCPR : 0;
  constexpr int NT = NW * 64;
  constexpr int LOADS = TILE_CHUNKS / NT;
  constexpr int VLOADS = VTILE_CHUNKS / NT;
  constexpr int NKK = HSP / 16;
  constexpr int NMT = VHSP / 32;
  constexpr int RW = NW * 32;
  static_assert(HSP % 64 == 0 && VHSP % 32 == 0 && VHSP <= HSP, "head sizes");
  static_assert(KT % 32 == 0 && TILE_CHUNKS % NT == 0 && VTILE_CHUNKS % NT == 0, "tile shape");
  static_assert(!SEP || VHSP % 64 == 0, "value rows: whole swizzle periods");
  static_assert(QREG % 16 == 0 && QREG <= HSP, "register part of the query");
  // LDS: [KV tile buffers | persistent query rows, channels >= QREG]. Before the
  // tile loop the buffer region (EARLY below: its last buffer) stages the
  // register part of the query.
  constexpr int QSTRIDE = QREG + 8;     // staged rows padded by 16 bytes against bank conflicts
  constexpr int QRS = HSP - QREG + 8;
  constexpr int BUF_BYTES = (TILE_CHUNKS + VTILE_CHUNKS) * 16;   // K rows, then (SEP) V rows
  // Tile buffers: NBUF - 1 tiles are in flight while one is computed. Three
  // when two workgroups still fit in a CU's 160 KB of LDS, else two.
  constexpr int NBUF_WANT = NW >= 4 ? PA_GEN_NBUF4 : PA_GEN_NBUF;
  constexpr int NBUF = (2 * NBUF_WANT * BUF_BYTES <= 150 * 1024) ? NBUF_WANT : 2;
  constexpr int PER = LOADS + VLOADS;   // copy instructions per wave and tile (vmcnt counts them)
  constexpr int QSTAGE_BYTES = RW * QSTRIDE * 2;
  // When the staged query fits in one tile buffer it is staged in the last
  // one, and the first NBUF - 1 tiles of a piece are issued before the query
  // loads (into the other buffers), so the two latencies overlap (the
  // one-wave decode instances).
  constexpr bool EARLY = QSTAGE_BYTES <= BUF_BYTES;
  constexpr int QSTAGE_OFF = EARLY ? (NBUF - 1) * BUF_BYTES : 0;
  constexpr int KV_BYTES = (NBUF * BUF_BYTES > QSTAGE_BYTES) ? NBUF * BUF_BYTES : QSTAGE_BYTES;
  constexpr int QREST_BYTES = (QREG < HSP) ? RW * QRS * 2 : 0;
  constexpr int LDS_BYTES = KV_BYTES + QREST_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

  __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[LDS_BYTES];

  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);   // wave index, scalar
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
  // Copies move groups of GK keys: group g of a tile (keys GK g .. GK g +
  // GK - 1) lies in one cache block (block_size >= 16, a power of two, and GK
  // divides 16), so one descriptor serves all its copy instructions; wave w
  // copies groups w, w + NW, ... Copy instruction i of a group fills LDS slots
  // 64 i .. 64 i + 63 of the group's rows. load_off[i]: byte offset, from the
  // group's first row, of the chunk the lane copies (chunks past the head, for
  // padded head sizes, get an offset past every descriptor and land as zeros).
  constexpr int GK = (KT / NW) < 16 ? (KT / NW) : 16;   // keys per copy group
  constexpr int KG = KT / GK;           // key groups per tile
  constexpr int GPW = KG / NW;          // groups per wave
  constexpr int IPG = GK * CPR / 64;    // K copy instructions per group
  constexpr int VIPG = SEP ? GK * VCPR / 64 : 0;
  static_assert(KG % NW == 0 && (GK * CPR) % 64 == 0 && (GK * VCPR) % 64 == 0 && GPW * IPG == LOADS &&
                GPW * VIPG == VLOADS, "copy split");
  // The LDS swizzle follows the key index within the tile (period 16); with
  // one group per wave that is GK w + kl, else (GK = 16) kl.
  const int swz0 = GPW == 1 ? GK * w : 0;
  uint32_t load_off[IPG];
#pragma unroll
  for (int i = 0; i < IPG; ++i) {
    const int pidx = i * 64 + lane;
    const int kl = pidx / CPR;
    const int lc = (pidx - kl * CPR) ^ lds_swizzle(swz0 + kl);
    load_off[i] = lc * 8 < p.hs ? (uint32_t)((kl * p.krs + lc * 8) * 2) : kOutOfRange;
  }
  uint32_t vload_off[VIPG > 0 ? VIPG : 1];
#pragma unroll
  for (int i = 0; i < VIPG; ++i) {
    const int pidx = i * 64 + lane;
    const int kl = pidx / VCPR;
    const int lc = (pidx - kl * VCPR) ^ lds_swizzle(swz0 + kl);
    vload_off[i] = lc * 8 < p.vhs ? (uint32_t)((kl * p.vrs + lc * 8) * 2) : kOutOfRange;
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
    const int past_b = t.past;

    const int rloc = w * 32 + l32;
    const bool row_ok = rloc < t.nrows;
    const int R = t.row0 + rloc;
    const int tq = R / p.H;
    const int pos = row_ok ? past_b + tq : -1;
    const int lo_row = p.window >= 0 ? max(0, pos - p.window) : 0;
    const bool wave_active = w * 32 < t.nrows;
    // Keys every row of this wave sees: [lo_max_w, pos_min_w] (wave-uniform).
    const int pos_min_w = past_b + (t.row0 + w * 32) / p.H;
    const int pos_max_w = past_b + (t.row0 + min(w * 32 + 31, t.nrows - 1)) / p.H;
    const int lo_max_w = p.window >= 0 ? max(0, pos_max_w - p.window) : 0;
    const int64_t qrow = head_row(p, t, R);

    // Copy KV tile `tile` into LDS buffer `bufi`: exactly PER copy
    // instructions per wave (vmcnt counts them), 16 bytes per lane, global ->
    // LDS directly. A group's descriptor covers its keys below kv_hi, so later
    // keys land as zeros; keys below kv_lo (the first tile of a windowed
    // range) take an out-of-range offset per lane.
    const uint32_t lds0 = lds_addr(lds_raw);
    // Groups [G0, G1) of the wave (GPW in all): a tile's copies may go out
    // in two parts, the second during the tile computation.
    auto issue_groups = [&](int tile, int bufi, auto G0, auto G1) {
      constexpr int g0 = decltype(G0)::value, g1 = decltype(G1)::value;
      const int key0 = tile * KT;
      int ids[GPW];
#pragma unroll
      for (int gi = g0; gi < g1; ++gi) {
        const int kg = key0 + GK * (gi * NW + w);
        ids[gi] = ld_uniform(p.bt + (int64_t)b * p.MB + min(kg >> p.bs_log2, p.MB - 1));
      }
      __builtin_amdgcn_sched_barrier(0);   // every block-id load goes out before the first use
#pragma unroll
      for (int gi = g0; gi < g1; ++gi) {
        const int g = gi * NW + w;
        const int kg = key0 + GK * g;                     // first key of the group
        const int nkeys = min(max(t.kv_hi - kg, 0), GK);
        const int64_t row0 = ((int64_t)clamp_block(ids[gi], p.nblk) << p.bs_log2) + (kg & ((1 << p.bs_log2) - 1));
        const uint32_t dst = lds0 + (uint32_t)(bufi * BUF_BYTES + g * GK * CPR * 16);
        const u32x4_t rk = rsrc_words_u(p.cache + row0 * p.krs + t.kvg * p.hs, (uint32_t)(nkeys * p.krs * 2));
        const bool lower = kg < t.kv_lo;
#pragma unroll
        for (int i = 0; i < IPG; ++i) {
          uint32_t off = load_off[i];
          if (lower) off = kg + (i * 64 + opaque_lane()) / CPR >= t.kv_lo ? off : kOutOfRange;
          copy16_to_lds(dst + i * 64 * 16, off, rk);
        }
        if constexpr (SEP) {
          const uint32_t vdst = lds0 + (uint32_t)(bufi * BUF_BYTES + (TILE_CHUNKS + g * GK * VCPR) * 16);
          const u32x4_t rv = rsrc_words_u(p.vcache + row0 * p.vrs + t.kvg * p.vhs, (uint32_t)(nkeys * p.vrs * 2));
#pragma unroll
          for (int i = 0; i < VIPG; ++i) {
            uint32_t off = vload_off[i];
            if (lower) off = kg + (i * 64 + opaque_lane()) / VCPR >= t.kv_lo ? off : kOutOfRange;
            copy16_to_lds(vdst + i * 64 * 16, off, rv);
          }
        }
      }
    };
    using IG0 = std::integral_constant<int, 0>;
    using IGH = std::integral_constant<int, GPW / 2>;
    using IGW = std::integral_constant<int, GPW>;
    auto issue = [&](int tile, int bufi) { issue_groups(tile, bufi, IG0{}, IGW{}); };

    if constexpr (EARLY) {
#pragma unroll
      for (int k = 0; k < NBUF - 1; ++k)
        if (tile_a + k < tile_b) issue(tile_a + k, k);
    }
    WaveState<DT, HSP, VHSP, KT, QREG> st;
    // Query rows of this wave, staged through LDS (free between pieces),
    // RoPE'd there, read back as fragments (row l32, channels 16 kk + 8 hi ..
    // + 8). Every global load of a phase is issued before the first use of
    // its result (a load-use loop would pay the memory latency per chunk).
    uint16_t* const qrest = (uint16_t*)(lds_raw + KV_BYTES) + w * 32 * QRS;
    {
      uint16_t* qs = (uint16_t*)(lds_raw + QSTAGE_OFF) + w * 32 * QSTRIDE;
      // element (r, c) of this wave's staged query rows
      auto qel = [&](int r, int c) -> uint16_t* { return c < QREG ? qs + r * QSTRIDE + c : qrest + r * QRS + (c - QREG); };
      constexpr int QCH = HSP / 8;
      // Lane-derived indices are formed here from an opaque lane id: hoisted
      // out of the piece loop they would be kept in spill slots.
      const int ln = opaque_lane();
      // RoPE: one task rotates 8 channels of a row: non-interleaved, channels
      // ro + 8 i .. + 8 with their partners half channels later (cos/sin
      // entries 8 i .. + 8); interleaved, the 4 pairs of channels
      // ro + 8 j .. + 8 (entries 4 j .. + 4). Tasks go four per lane at a
      // time. The table entries of the first four tasks are loaded together
      // with the query rows (they depend only on the rows' positions), so
      // the staging waits for memory once.
      const int half = p.rd >> 1;
      // (at least 1: without rotary channels no task exists, and rr below divides by it)
      const int per_row = max(p.interleaved ? p.rd / 8 : half / 8, 1);
      const int ntask = p.do_rotary ? 32 * per_row : 0;
      u32x4_t cv[4], sv[4];
      int rr[4], gg[4];
      bool ok[4];
      auto load_tables = [&](int tb) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int task = tb + k * 64 + ln;
          rr[k] = task / per_row;
          gg[k] = task - rr[k] * per_row;
          ok[k] = task < ntask && w * 32 + rr[k] < t.nrows;
          cv[k] = sv[k] = u32x4_t{0u, 0u, 0u, 0u};
          if (ok[k]) {
            const int posr = past_b + (t.row0 + w * 32 + rr[k]) / p.H;
            const int64_t e0 = min(max((int64_t)posr, (int64_t)0), p.prow - 1) * half;
            if (p.interleaved) {
              const u32x2_t c2 = *(const u32x2_t*)(p.cos_t + e0 + 4 * gg[k]);
              const u32x2_t s2 = *(const u32x2_t*)(p.sin_t + e0 + 4 * gg[k]);
              cv[k] = u32x4_t{c2[0], c2[1], 0u, 0u};
              sv[k] = u32x4_t{s2[0], s2[1], 0u, 0u};
            } else {
              cv[k] = *(const u32x4_t*)(p.cos_t + e0 + 8 * gg[k]);
              sv[k] = *(const u32x4_t*)(p.sin_t + e0 + 8 * gg[k]);
            }
          }
        }
      };
      load_tables(0);
      // The query rows: 32 rows x QCH chunks over 64 lanes, every load in
      // flight at once.
      constexpr int NQL = QCH / 2;
      {
        u32x4_t qv[NQL];
#pragma unroll
        for (int q = 0; q < NQL; ++q) {
          const int idx = q * 64 + ln;
          const int r = idx / QCH;
          const int c0 = (idx - r * QCH) * 8;
          qv[q] = u32x4_t{0u, 0u, 0u, 0u};
          if (w * 32 + r < t.nrows && c0 < p.hs)
            qv[q] = *(const u32x4_t*)(p.query + head_row(p, t, t.row0 + w * 32 + r) * p.hs + c0);
        }
#pragma unroll
        for (int q = 0; q < NQL; ++q) {
          const int idx = q * 64 + ln;
          const int r = idx / QCH;
          *(u32x4_t*)qel(r, (idx - r * QCH) * 8) = qv[q];
        }
      }
      __syncthreads();
      for (int tb = 0; tb < ntask; tb += 4 * 64) {
        if (tb > 0) load_tables(tb);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (!ok[k]) continue;
          float c[8], sn[8];
          unpack8<DT>(cv[k], c);
          unpack8<DT>(sv[k], sn);
          if (p.interleaved) {
            uint16_t* e = qel(rr[k], p.ro + 8 * gg[k]);
            float x[8];
            unpack8<DT>(*(const u32x4_t*)e, x);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              const float xe = x[2 * m], xo = x[2 * m + 1];
              x[2 * m] = xe * c[m] - xo * sn[m];
              x[2 * m + 1] = xo * c[m] + xe * sn[m];
            }
            *(u32x4_t*)e = pack8<DT>(x);
          } else {
            uint16_t* e1 = qel(rr[k], p.ro + 8 * gg[k]);
            uint16_t* e2 = qel(rr[k], p.ro + 8 * gg[k] + half);
            float x1[8], x2[8], y1[8], y2[8];
            unpack8<DT>(*(const u32x4_t*)e1, x1);
            unpack8<DT>(*(const u32x4_t*)e2, x2);
#pragma unroll
            for (int m = 0; m < 8; ++m) {
              y1[m] = x1[m] * c[m] - x2[m] * sn[m];
              y2[m] = x2[m] * c[m] + x1[m] * sn[m];
            }
            *(u32x4_t*)e1 = pack8<DT>(y1);
            *(u32x4_t*)e2 = pack8<DT>(y2);
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < QREG / 16; ++kk)
        st.qf[kk] = *(const u32x4_t*)(qs + l32 * QSTRIDE + 16 * kk + 8 * hi);
      __syncthreads();
    }
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) st.o[mt] = f32x16_t{};
    st.m_run = -INFINITY;
    st.l_run = 0.0f;

    // Ring of NBUF buffers: tile tt sits in buffer (tt - tile_a) % NBUF; the
    // first NBUF - 1 tiles go out before the loop (EARLY: before the query
    // staging), and iteration tt, once every wave has passed its barrier (so
    // the buffer of tile tt - 1 is free), issues tile tt + NBUF - 1 into that
    // buffer.
    if constexpr (!EARLY) {
#pragma unroll
      for (int k = 0; k < NBUF - 1; ++k)
        if (tile_a + k < tile_b) issue(tile_a + k, k);
    }
    for (int tt = tile_a; tt < tile_b; ++tt) {
      const int bufi = (tt - tile_a) % NBUF;
      // This wave's copies of tile tt are done once at most (tiles issued
      // after it) * PER copies remain in flight; the barrier then makes every
      // wave's copies of tile tt visible.
      if constexpr (NW >= 4 && PA_GEN_PRIO == 0) {
        // Two workgroups share a CU (one wave of each per SIMD). With equal
        // priorities the SIMDs favour the older wave, so the workgroups of
        // the grid's first half ran ahead and those of the second half
        // finished last; the priority alternates every tile, in opposite
        // phase in the two halves, so both share the SIMDs evenly.
        if (((tt & 1) != 0) != (blockIdx.x >= gridDim.x / 2)) asm volatile("s_setprio 1");
        else asm volatile("s_setprio 0");
      }
      vm_wait_tiles<PER, NBUF - 2>(min(NBUF - 2, tile_b - 1 - tt));
      lds_barrier();
      // A CU stalls vector-memory issue once some 48 KB of loads are in
      // flight: a whole tile's copies at once would hold the wave there,
      // so the groups of the second half go out after the QK MFMAs.
      const bool next = tt + NBUF - 1 < tile_b;
      const int nbuf = (tt + NBUF - 1 - tile_a) % NBUF;
      if (next) issue_groups(tt + NBUF - 1, nbuf, IG0{}, IGH{});
      {
        // Every wave computes, also one without rows in this tile (its rows
        // are zero queries and are never stored): a branch here would make
        // the accumulators loop-carried through two paths, and the compiler
        // then copies them at every iteration.
        const uint8_t* buf = lds_raw + bufi * BUF_BYTES;
        const bool full = wave_active && tt * KT >= lo_max_w && tt * KT + KT - 1 <= pos_min_w;
        tile_compute<DT, HSP, VHSP, KT, QREG, VCPR, GEN>(st, buf, buf + (SEP ? TILE_CHUNKS * 16 : 0), qrest, tt * KT,
                                                    pos, lo_row, softcap_on, full, p, [&]() {
                                                      if (next) issue_groups(tt + NBUF - 1, nbuf, IGH{}, IGW{});
                                                    });
      }
    }
    __syncthreads();

    const float l_tot = st.l_run + __shfl_xor(st.l_run, 32);
    // A whole query tile writes its output rows. A split-KV piece writes its
    // own normalised output acc / l into its partial slot (element type
    // PartT, rows padded to VHSP channels) and (m, l) in float32; the combine
    // merges the pieces.
    if (row_ok) {
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
      if (whole) {
        uint16_t* const orow = p.out + qrow * p.vhs;
        if (p.vhs == VHSP) {
          // Lane writes channels mt*32 + hi*4 + 8*grp .. + 3 of its row: one
          // base address, immediate offsets.
          uint16_t* ob = orow + hi * 4;
#pragma unroll
          for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
              const uint32_t e0 = DT::from_f32(st.o[mt][4 * grp + 0] * inv);
              const uint32_t e1 = DT::from_f32(st.o[mt][4 * grp + 1] * inv);
              const uint32_t e2 = DT::from_f32(st.o[mt][4 * grp + 2] * inv);
              const uint32_t e3 = DT::from_f32(st.o[mt][4 * grp + 3] * inv);
              *(u32x2_t*)(ob + mt * 32 + 8 * grp) = u32x2_t{e0 | (e1 << 16), e2 | (e3 << 16)};
            }
          }
        } else {
          for (int mt = 0; mt < NMT; ++mt) {
            for (int e = 0; e < 16; ++e) {
              const int c = mt * 32 + hi * 4 + 8 * (e >> 2) + (e & 3);
              if (c < p.vhs) orow[c] = (uint16_t)DT::from_f32(st.o[mt][e] * inv);
            }
          }
        }
      } else {
        // The workgroup's first piece goes to slot wr, a later one to G + tile.
        const int64_t slot = i == i_first ? (int64_t)wr : (int64_t)gridDim.x + i;
        if (hi == 0) {
          float* ml = p.part_ml + (slot * RW + rloc) * 2;
          ml[0] = st.m_run;
          ml[1] = l_tot;
        }
        const int64_t prow = slot * p.part_slot + (int64_t)rloc * p.part_row + hi * 4;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
          for (int grp = 0; grp < 4; ++grp) {
            const int64_t off = prow + mt * 32 + 8 * grp;
            const float x0 = st.o[mt][4 * grp + 0] * inv, x1 = st.o[mt][4 * grp + 1] * inv;
            const float x2 = st.o[mt][4 * grp + 2] * inv, x3 = st.o[mt][4 * grp + 3] * inv;
            if constexpr (PartF32<DT>::value) {
              *(f32x4_t*)((float*)p.part_o + off) = f32x4_t{x0, x1, x2, x3};
            } else {
              *(u32x2_t*)((uint16_t*)p.part_o + off) =
                  u32x2_t{DT::pack2(x0, x1), DT::pack2(x2, x3)};
            }
          }
        }
      }
    }
    u = ub;
    ++i;
  }

#endif  // __HIP_DEVICE_COMPILE__
}

// Partial slot of piece q of a split query tile t (the workgroups w_first,
// w_first + 1, ...): a workgroup stores its first piece in slot w and a later
// piece (only ever piece 0 of its tile) in slot G + tile, which the schedule
// records as the tile's part_base.
__device__ __forceinline__ int64_t piece_slot(const MTile& t, int q) {
  return q == 0 ? (int64_t)t.part_base : (int64_t)t.w_first + q;
}

// Merge the partials of every query tile that several workgroups processed
// (piece q's partial at slot piece_slot(t, q)). Piece i of a row holds its normalised output o_i = acc_i / l_i (bfloat16
// for bfloat16 outputs, else float32: PartF32), its running max m_i (log2
// domain) and denominator l_i; with
// M = max_i m_i and c_i = 2^(m_i - M) l_i, out = sum_i c_i o_i / sum_i c_i
// (float32), rounded to nearest even.
// Grid: (query tiles, ceil(RW / ROWS)) of 256 threads, ROWS rows per block.
// TPR threads share a row; thread j of a row owns the 8-channel groups j,
// j + TPR, j + 2 TPR, ... (so each load instruction covers contiguous bytes
// of a row). Every thread forms its row's weights itself from the (m, l)
// pairs. Up to QA pieces: the pairs and all slice loads go out together (one
// round trip). More pieces: the pairs are read QM pieces at a time, then the
// slices QA pieces at a time with all their 16-byte loads in flight together.
// MANY: the launch expects many pieces per tile (short decode batches), so
// rows of one 8-channel group take 16 pieces per round trip (the registers
// this holds would lower the occupancy of launches with few pieces).
template <int VHSP, bool MANY = false>
struct CombineShape {
  static constexpr int TPR = (VHSP / 8) < PA_COMB_TPR ? (VHSP / 8) : PA_COMB_TPR;   // threads per row
  static constexpr int CPT = VHSP / TPR;                          // channels per thread (multiple of 8)
  static constexpr int ROWS = 256 / TPR;                          // rows per block
  static constexpr int NV = CPT / 8;
  static constexpr int QA = (MANY && NV == 1) ? 16 : (NV <= 2 ? PA_COMB_QA : 4);   // pieces per round trip
};

template <typename DT, int VHSP, int RW, bool MANY = false>
__global__ __launch_bounds__(256) void combine_kernel(AttnParams p) {
  using CS = CombineShape<VHSP, MANY>;
  constexpr int TPR = CS::TPR;
  constexpr int CPT = CS::CPT;
  constexpr int ROWS = CS::ROWS;
  constexpr int NV = CS::NV;
  constexpr int QM = 8;                                    // pieces per batch of (m, l) loads
  constexpr int QA = CS::QA;                               // pieces per batch of slice loads
  static_assert(CPT % 8 == 0 && CPT * TPR == VHSP, "channel split");
  const int i = blockIdx.x;
  if (i >= ld_uniform(p.header + 1)) return;
  const MTile t = ld_uniform_tile(p.mt + i);
  if (t.npieces <= 1) return;
  const int r0 = blockIdx.y * ROWS;
  if (r0 >= t.nrows) return;
  const int nq = t.npieces;
  {
    const int rr = threadIdx.x / TPR;
    const int r = r0 + rr;
    if (r >= t.nrows) return;
    const int c0 = (threadIdx.x % TPR) * 8;                 // channel of group 0; group v at c0 + 8 TPR v
    if (c0 >= p.vhs) return;
    // Piece q's (m, l) and slice (16-byte aligned: row and slot strides are
    // multiples of 16 bytes).
    auto ml_of = [&](int q) -> const float* { return p.part_ml + (piece_slot(t, q) * RW + r) * 2; };
    auto po_of = [&](int q) -> int64_t { return piece_slot(t, q) * p.part_slot + (int64_t)r * p.part_row + c0; };
    float acc[NV][8];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[v][e] = 0.0f;
    auto add = [&](float wgt, const float (&a)[NV][8]) {
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[v][e] += wgt * a[v][e];
    };
    if (nq <= QA) {
      // Up to QA pieces (the usual case): the (m, l) pairs and every slice
      // load are issued together, one memory round trip per row.
      float a[QA][NV][8];
      float m[QA], l[QA];
#pragma unroll
      for (int k = 0; k < QA; ++k) {
        // Pieces past nq (uniform over the block) load nothing.
        m[k] = -INFINITY;
        l[k] = 0.0f;
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
          for (int e = 0; e < 8; ++e) a[k][v][e] = 0.0f;
        if (k < nq) {
          m[k] = ml_of(k)[0];
          l[k] = ml_of(k)[1];
#pragma unroll
          for (int v = 0; v < NV; ++v) load_part8<DT>(p.part_o, po_of(k) + 8 * TPR * v, a[k][v]);
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int k = 0; k < QA; ++k) mx = fmaxf(mx, m[k]);
      float cq[QA], den = 0.0f;
#pragma unroll
      for (int k = 0; k < QA; ++k) {
        cq[k] = m[k] == -INFINITY ? 0.0f : fast_exp2(m[k] - mx) * l[k];
        den += cq[k];
      }
      const float inv = den > 0.0f ? 1.0f / den : 0.0f;
#pragma unroll
      for (int k = 0; k < QA; ++k) add(cq[k] * inv, a[k]);
    } else {
      // Reference max and denominator: one batch of (m, l) loads per QM pieces.
      float mx = -INFINITY, den = 0.0f;
      for (int q0 = 0; q0 < nq; q0 += QM) {
        float m[QM], l[QM];
#pragma unroll
        for (int k = 0; k < QM; ++k) {
          const bool ok = q0 + k < nq;
          m[k] = ok ? ml_of(q0 + k)[0] : -INFINITY;
          l[k] = ok ? ml_of(q0 + k)[1] : 0.0f;
        }
        float bm = -INFINITY;
#pragma unroll
        for (int k = 0; k < QM; ++k) bm = fmaxf(bm, m[k]);
        const float nm = fmaxf(mx, bm);
        den = (mx == -INFINITY) ? 0.0f : den * fast_exp2(mx - nm);
#pragma unroll
        for (int k = 0; k < QM; ++k) den += (m[k] == -INFINITY) ? 0.0f : fast_exp2(m[k] - nm) * l[k];
        mx = nm;
      }
      const float inv = den > 0.0f ? 1.0f / den : 0.0f;
      // Weighted sum of the row slices.
      for (int q0 = 0; q0 < nq; q0 += QA) {
        float a[QA][NV][8];
        float wq[QA];
#pragma unroll
        for (int k = 0; k < QA; ++k) {
          const bool ok = q0 + k < nq;
          const int q = ok ? q0 + k : q0;
#pragma unroll
          for (int v = 0; v < NV; ++v) load_part8<DT>(p.part_o, po_of(q) + 8 * TPR * v, a[k][v]);
          const float m = ml_of(q)[0], l = ml_of(q)[1];
          wq[k] = (!ok || m == -INFINITY) ? 0.0f : fast_exp2(m - mx) * l * inv;
        }
#pragma unroll
        for (int k = 0; k < QA; ++k) add(wq[k], a[k]);
      }
    }
    uint16_t* orow = p.out + head_row(p, t, t.row0 + r) * p.vhs + c0;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int c = c0 + 8 * TPR * v;
      if ((p.vhs & 7) == 0) {
        if (c < p.vhs) *(u32x4_t*)(orow + 8 * TPR * v) = pack8<DT>(acc[v]);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (c + k < p.vhs) orow[8 * TPR * v + k] = (uint16_t)DT::from_f32(acc[v][k]);
      }
    }
  }
}

// Launches the attention kernel (events ev[0] / ev[1] recorded around it when
// ev is non-null) and, when `combine`, the split-KV combine over `cgrid` query tiles.
typedef hipError_t (*AttnLaunchFn)(const AttnParams&, int, bool, int, hipStream_t, const hipEvent_t*);
typedef hipError_t (*AttnOccFn)(int*);

}  // namespace pa

// Instance names: LAY is lat (V = leading part of the latent row) or sep (separate
// value cache, grouped-query heads).
#define PA_ATTN_FN(LAY, DTN, HSP, VHSP, NW, KT, SUF) attn_##LAY##_##DTN##_##HSP##_##VHSP##_##NW##_##KT##_##SUF
#define PA_SEP_lat false
#define PA_SEP_sep true
#define PA_DEFINE_ATTN_INSTANCE(LAY, DT, DTN, HSP, VHSP, NW, KT, QREG)                                      \
  namespace pa {                                                                                          \
  hipError_t PA_ATTN_FN(LAY, DTN, HSP, VHSP, NW, KT, occ)(int* n) {                                       \
    void (*fn)(AttnParams) = attn_kernel<DT, HSP, VHSP, NW, KT, QREG, PA_SEP_##LAY, false>;               \
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, reinterpret_cast<const void*>(fn), NW * 64, 0);   \
  }                                                                                                       \
  hipError_t PA_ATTN_FN(LAY, DTN, HSP, VHSP, NW, KT, launch)(const AttnParams& p, int grid, bool combine,  \
                                                             int cgrid, hipStream_t s, const hipEvent_t* ev) { \
    hipError_t e = ev ? hipEventRecord(ev[0], s) : hipSuccess;                                            \
    if (e != hipSuccess) return e;                                                                        \
    if (p.softcap > 0.0f || !(p.scale_log2 > 0.0f))                                                       \
      attn_kernel<DT, HSP, VHSP, NW, KT, QREG, PA_SEP_##LAY, true><<<grid, NW * 64, 0, s>>>(p);           \
    else                                                                                                  \
      attn_kernel<DT, HSP, VHSP, NW, KT, QREG, PA_SEP_##LAY, false><<<grid, NW * 64, 0, s>>>(p);          \
    e = hipGetLastError();                                                                                \
    if (e == hipSuccess && ev) e = hipEventRecord(ev[1], s);                                              \
    if (e != hipSuccess || !combine) return e;                                                            \
    {                                                                                                     \
      const dim3 cg(cgrid, (NW * 32 + CombineShape<VHSP>::ROWS - 1) / CombineShape<VHSP>::ROWS);          \
      if (CombineShape<VHSP>::NV == 1 && p.many_pieces) combine_kernel<DT, VHSP, NW * 32, true><<<cg, 256, 0, s>>>(p); \
      else combine_kernel<DT, VHSP, NW * 32><<<cg, 256, 0, s>>>(p);                                       \
    }                                                                                                     \
    return hipGetLastError();                                                                             \
  }                                                                                                       \
  }
#define PA_DECLARE_ATTN_INSTANCE(LAY, DTN, HSP, VHSP, NW, KT)                                                   \
  hipError_t PA_ATTN_FN(LAY, DTN, HSP, VHSP, NW, KT, launch)(const AttnParams&, int, bool, int, hipStream_t,    \
                                                            const hipEvent_t*);                                 \
  hipError_t PA_ATTN_FN(LAY, DTN, HSP, VHSP, NW, KT, occ)(int*);
