// On-device work scheduler for the read phase, instance table, workspace plan
// and launch sequence (scheduler -> attention -> combine) on the caller's stream.
//
// The launch geometry depends only on host-known shapes (token count, batch,
// compute units); everything that depends on sequence lengths is derived on
// the device from cumulative_sequence_length / past_seqlens, with no readback
// (docs.rs page "onnx-runtime-ep-cuda src/kernels/paged_attention.rs", module
// comment "Capture safety": geometry fixed by tensor shapes, positions and
// blocks resolved on device).
#include "pa_attn.cuh"
#include "pa_write.cuh"

#include <algorithm>
#include <mutex>
#include <map>
#include <tuple>

namespace pa {

struct SchedParams {
  const int32_t* cumseq;
  const int32_t* past;
  int B, H, RW, KT, window, grid, split_kv;
  int kvh;           // key/value heads: each sequence is scheduled once per head (H = query heads per head)
  int max_pos;       // max_blocks_per_seq * block_size: past lengths are clamped to it
  int piece_units;   // virtual KV tiles charged at the start of every query tile
  int min_units;     // split-KV: fewest (virtual) units a workgroup's range may hold
  // Query pre-pass (blocks 1.., four-wave 576 kernel): the query with RoPE
  // applied, in the attention kernel's fragment order (qfrag, [T * H][hsp]).
  const uint16_t* query;
  const uint16_t* cos_t;
  const uint16_t* sin_t;
  uint16_t* qfrag;
  int hsp;
  int64_t T, prow;
  int hs, ro, rd, interleaved, dtype;
  int64_t max_mtiles, part_cap;
  int32_t* header;
  int32_t* wg_range;
  int32_t* wg_tile;
  int32_t* sched;    // global scratch for the arrays below when they exceed kSchedLdsInts
  MTile* mt;
  int rope_blocks;   // blocks 1 .. rope_blocks: the query pre-pass
  // Fused call (write phase in the same launch): blocks wblock0 .. wblock0 +
  // wblocks - 1 write token rows 4 (block - wblock0) .. + 3, one per wave,
  // from wkey into wcache (wslots cache rows); wblocks = 0 otherwise.
  // In the separate layout rows T .. 2T - 1 are the value rows (wval, wvcache).
  const uint16_t* wkey;
  const int32_t* wslot;
  uint16_t* wcache;
  const uint16_t* wval;
  uint16_t* wvcache;
  int64_t wslots;
  int wblock0, wblocks, vhs;
};

constexpr int kSchedThreads = 256;

// Exclusive prefix sum over n values get(i) (32-bit; every total here is an
// index below 2^31), written with put(i, prefix); returns the total. Every
// thread of the block must call it. Per chunk of kSchedThreads values: a
// shuffle scan inside each wave, then every thread adds the totals of the
// waves before its own (read from LDS in parallel, no serial pass).
template <typename Get, typename Put>
__device__ int32_t block_exclusive_scan(int64_t n, Get get, Put put) {
  constexpr int NWV = kSchedThreads / 64;
  __shared__ int32_t wave_sums[NWV];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t carry = 0;
  for (int64_t base = 0; base < n; base += kSchedThreads) {
    const int64_t idx = base + threadIdx.x;
    const int32_t v = idx < n ? get(idx) : 0;
    int32_t x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t y = __shfl_up(x, d);
      if (lane >= d) x += y;
    }
    if (lane == 63) wave_sums[wave] = x;
    __syncthreads();
    int32_t before = 0, total = 0;
#pragma unroll
    for (int k = 0; k < NWV; ++k) {
      const int32_t ws = wave_sums[k];
      before += k < wave ? ws : 0;
      total += ws;
    }
    if (idx < n) put(idx, carry + before + x - v);
    carry += total;
    __syncthreads();
  }
  return carry;
}

// Blocks 1.. of the schedule launch: the query in the four-wave kernel's
// fragment order, RoPE applied (float32 math, nearest-even rounding; the same
// rotation the write phase applies to key rows). Each sequence's rows are cut
// into blocks of 32 (the rows one wave holds); a block whose first row is R0
// and which has nv rows keeps the span [R0, R0 + nv) * hsp and stores 8-channel
// chunk c of its row l (zero past hs) at chunk c * nv + l, so the wave reads
// k-step s (chunks 2 s and 2 s + 1 of every row) as one contiguous run of
// 32 nv bytes.
//
// The copy is a transpose through LDS, kPreRows consecutive query rows at a
// time (whatever blocks they belong to): their contiguous bytes are loaded
// with coalesced 16-byte loads into LDS rows padded to an odd number of
// chunks, the rotary chunks are rotated there, and each chunk is stored to its
// place by threads that take consecutive rows of one channel chunk, so the
// stores of a block's rows are contiguous runs as well. `cum` and `pst` are
// cumulative_sequence_length and past_seqlens (staged in LDS when they fit).
// A row whose token the sequence bounds do not place inside [0, T) (only a
// violated precondition does that) is not stored.
constexpr int kPreRows = 32;
constexpr int kSchedLdsBytes = 40832;   // transpose buffer and staging; with the scan sums, four blocks per CU
constexpr int kPreMaxCpr = 72;                                       // chunks per row of a 576-wide copy
constexpr int kPreItems = (kPreRows * kPreMaxCpr + kSchedThreads - 1) / kSchedThreads;   // chunks per thread
constexpr int kPreTBytes = kPreRows * (kPreMaxCpr | 1) * 16;         // transpose buffer
// Per-row placement, behind the transpose buffer: first destination chunk of
// the row's column 0 (-1: not placed), its block's row count, position.
struct PreRow {
  int64_t dst0;
  int32_t nv, pos;
};
constexpr int kPreRowBytes = kPreRows * (int)sizeof(PreRow);

template <typename DT>
__device__ void query_frag_rows(const SchedParams& p, int64_t R_base, uint8_t* lds, const int32_t* cum,
                                const int32_t* pst) {
  const int cpr = p.hsp >> 3;                          // chunks per row of the copy (<= kPreMaxCpr)
  const int qcpr = p.hs >> 3;                          // chunks per query row
  const int pitch = cpr | 1;                           // LDS row pitch in chunks (odd: conflict-free columns)
  const int nr = (int)min((int64_t)kPreRows, p.T * p.H - R_base);
  if (cpr > kPreMaxCpr) return;                        // only the 576-wide copy exists
  PreRow* const rows = (PreRow*)(lds + kPreTBytes);
  auto at = [&](int r, int c) -> u32x4_t* { return (u32x4_t*)(lds + (r * pitch + c) * 16); };
  // All loads of the group in flight together (chunk k of the contiguous span).
  const u32x4_t* src = (const u32x4_t*)(p.query + R_base * p.hs);
  u32x4_t v[kPreItems];
#pragma unroll
  for (int q = 0; q < kPreItems; ++q) {
    const int k = q * kSchedThreads + threadIdx.x;
    const int r = k / cpr, c = k - r * cpr;
    v[q] = (r < nr && c < qcpr) ? src[r * qcpr + c] : u32x4_t{0u, 0u, 0u, 0u};
  }
  // Meanwhile the rows' placement: block of 32 rows within the row's sequence.
  if ((int)threadIdx.x < nr) {
    const int64_t R = R_base + threadIdx.x;
    const int64_t tok = R / p.H;
    const int b = find_seq(cum, p.B, tok);
    const int64_t lo = cum[b], hi = cum[b + 1];
    PreRow pr;
    pr.dst0 = -1;
    pr.nv = 0;
    pr.pos = 0;
    if (0 <= lo && lo <= tok && tok < hi && hi <= p.T) {
      const int64_t s0 = lo * p.H;                     // the sequence's first row
      const int64_t k32 = (R - s0) & ~(int64_t)31;     // first row of R's block, within the sequence
      const int64_t R0 = s0 + k32;
      pr.nv = (int)min((int64_t)32, (hi - lo) * p.H - k32);
      pr.dst0 = R0 * cpr + (R - R0);
      pr.pos = (int)min(max((int64_t)pst[b] + (tok - lo), (int64_t)0), p.prow - 1);
    }
    rows[threadIdx.x] = pr;
  }
#pragma unroll
  for (int q = 0; q < kPreItems; ++q) {
    const int k = q * kSchedThreads + threadIdx.x;
    const int r = k / cpr, c = k - r * cpr;
    if (r < nr) *at(r, c) = v[q];
  }
  __syncthreads();
  if (p.rd > 0) {
    // Non-interleaved: one thread per (row, pair of chunks c, c + rd/16);
    // interleaved: one per (row, rotary chunk), the pairs inside it.
    const int half = p.rd >> 1;
    const int per_row = p.interleaved ? p.rd >> 3 : p.rd >> 4;
    for (int k = threadIdx.x; k < nr * per_row; k += kSchedThreads) {
      const int r = k / per_row, j = k - r * per_row;
      const PreRow pr = rows[r];
      if (pr.dst0 < 0) continue;
      const int c = (p.ro >> 3) + j;
      float x[8];
      unpack8<DT>(*at(r, c), x);
      if (p.interleaved) {
        const int64_t i0 = (int64_t)pr.pos * half + ((c * 8 - p.ro) >> 1);
        const u32x2_t cv = *(const u32x2_t*)(p.cos_t + i0);
        const u32x2_t sv = *(const u32x2_t*)(p.sin_t + i0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t cw = cv[e >> 1], sw = sv[e >> 1];
          const float co = DT::to_f32((e & 1) ? (cw >> 16) : (cw & 0xFFFFu));
          const float si = DT::to_f32((e & 1) ? (sw >> 16) : (sw & 0xFFFFu));
          const float xe = x[2 * e], xo = x[2 * e + 1];
          x[2 * e] = xe * co - xo * si;
          x[2 * e + 1] = xo * co + xe * si;
        }
        *at(r, c) = pack8<DT>(x);
      } else {
        const int cp = c + (half >> 3);                 // partner chunk, channel + rd/2
        float xp[8], c8[8], s8[8];
        unpack8<DT>(*at(r, cp), xp);
        const int64_t i0 = (int64_t)pr.pos * half + (c * 8 - p.ro);
        unpack8<DT>(*(const u32x4_t*)(p.cos_t + i0), c8);
        unpack8<DT>(*(const u32x4_t*)(p.sin_t + i0), s8);
        float y[8], yp[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          y[e] = x[e] * c8[e] - xp[e] * s8[e];
          yp[e] = xp[e] * c8[e] + x[e] * s8[e];
        }
        *at(r, c) = pack8<DT>(y);
        *at(r, cp) = pack8<DT>(yp);
      }
    }
    __syncthreads();
  }
  // Stores: consecutive threads take consecutive rows of one channel chunk.
#pragma unroll
  for (int q = 0; q < kPreItems; ++q) {
    const int k = q * kSchedThreads + threadIdx.x;
    if (k >= nr * cpr) continue;
    const int c = k / nr, r = k - c * nr;
    const PreRow pr = rows[r];
    if (pr.dst0 < 0) continue;
    *(u32x4_t*)(p.qfrag + (pr.dst0 + (int64_t)c * pr.nv) * 8) = *at(r, c);
  }
  __syncthreads();   // LDS free for the next rows
}

// Block 0 of the schedule launch builds the schedule. Its working arrays
// (per sequence: token range, past length, first query tile; per query tile:
// sequence, rows, key range, first work unit) live in LDS when they fit
// (IN_LDS is a template argument, so the compiler sees the LDS array), else
// in the workspace. The outputs are written once, in the last phase, where no
// barrier follows: a global store before a barrier would make the barrier
// wait for it.
//
// Work units are the KV tiles of every query tile, laid end to end. With
// split-KV on, each query tile is charged piece_units virtual units before
// its first real one (the cost of the query load and the epilogue a piece
// adds), and the virtual line of Uv = U + piece_units * M units is cut at
// x(w) = floor(w Uv / G) for w = 0..G (x(w) = min(w, Uv) when Uv < G); a cut
// inside a tile's virtual prefix falls on the tile's first unit. Because the
// cuts have a closed form, every query tile finds the workgroups whose cuts
// land in its range by counting, not searching: cnt(v), the number of cuts
// below v, gives the first workgroup W_i of tile i's range, the number P_i of
// cuts in its virtual prefix, and so the first workgroup that holds one of
// its units (W_i + P_i - 1) and the last (W_{i+1} - 1).
//
// Partial slots (split tiles only): a workgroup stores the partial result of
// its first piece in slot w and that of a later piece of query tile i in slot
// G + i (only a workgroup's first and last pieces can be partial, and a tile
// starts inside at most one workgroup's range), so at most G + M slots.
constexpr int kSchedLdsInts = kSchedLdsBytes / 4;

__host__ __device__ inline int64_t sched_ints(int B, int64_t max_mtiles, int /*grid*/) {
  return 4 * (int64_t)B + 1 + 6 * max_mtiles + 1;
}

template <bool IN_LDS>
__device__ __forceinline__ void schedule_build(const SchedParams& p, int32_t* lds_arr) {
  // Scheduled sequences: (sequence b, key/value head g) as sb = b * kvh + g;
  // in the latent layout kvh = 1 and sb = b.
  const int SB = p.B * p.kvh;
  int32_t* const base = IN_LDS ? lds_arr : p.sched;
  int32_t* const tlo = base;                           // [SB] first token of each sequence
  int32_t* const thi = tlo + SB;                       // [SB] end token
  int32_t* const pst = thi + SB;                       // [SB] past length
  int32_t* const sbase = pst + SB;                     // [SB + 1] first query tile of each sequence
  int32_t* const u0 = sbase + (SB + 1);                // [max_mtiles + 1] KV tiles, then first unit
  int32_t* const tb = u0 + (p.max_mtiles + 1);         // [max_mtiles] sequence of each tile
  int32_t* const trow = tb + p.max_mtiles;             // [max_mtiles] first row, rows (2 x)
  int32_t* const tkv = trow + 2 * p.max_mtiles;        // [max_mtiles] kv_lo, kv_hi (2 x)

  // A. Sequence bounds and past lengths, forced into the ranges the
  // preconditions promise (a violated precondition then gives unspecified
  // values but no access outside the caller's buffers): token ranges clamped
  // into [0, T] (empty when reversed), past lengths into [0, MB * bs].
  for (int sb = threadIdx.x; sb < SB; sb += kSchedThreads) {
    const int b = sb / p.kvh;
    const int32_t lo = (int32_t)min(max((int64_t)p.cumseq[b], (int64_t)0), p.T);
    const int32_t hi = (int32_t)min(max((int64_t)p.cumseq[b + 1], (int64_t)lo), p.T);
    tlo[sb] = lo;
    thi[sb] = hi;
    pst[sb] = min(max(p.past[b], 0), p.max_pos);
  }
  __syncthreads();
  // B. Query tiles per sequence, prefix-summed into sbase.
  const int64_t M_all = block_exclusive_scan(
      SB,
      [&](int64_t b) -> int32_t { return (int32_t)(((int64_t)(thi[b] - tlo[b]) * p.H + p.RW - 1) / p.RW); },
      [&](int64_t b, int32_t v) { sbase[b] = v; });
  // At most max_mtiles: the clamped ranges hold at most T tokens in at most
  // min(B, T) non-empty sequences, each scheduled kvh times.
  const int M = (int)min(M_all, p.max_mtiles);
  if (threadIdx.x == 0) sbase[SB] = (int32_t)M_all;
  __syncthreads();
  // C. Every query tile: its sequence (last b with sbase[b] <= i), rows, key
  // range and KV tile count; then the count's prefix sum into u0.
  for (int i = threadIdx.x; i < M; i += kSchedThreads) {
    int lo = 0, hi = SB - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sbase[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int rows = (thi[b] - tlo[b]) * p.H;
    const int row0 = (i - sbase[b]) * p.RW;
    const int nrows = min(p.RW, rows - row0);
    const int pos0 = pst[b] + row0 / p.H;
    const int pos1 = pst[b] + (row0 + nrows - 1) / p.H;
    const int kv_hi = pos1 + 1;
    const int kv_lo = p.window >= 0 ? max(0, pos0 - p.window) : 0;
    tb[i] = b;
    trow[2 * i] = row0;
    trow[2 * i + 1] = nrows;
    tkv[2 * i] = kv_lo;
    tkv[2 * i + 1] = kv_hi;
    u0[i] = (kv_hi + p.KT - 1) / p.KT - kv_lo / p.KT;
  }
  __syncthreads();
  const int64_t U = block_exclusive_scan(
      M, [&](int64_t i) -> int32_t { return u0[i]; }, [&](int64_t i, int32_t v) { u0[i] = v; });
  if (threadIdx.x == 0) u0[M] = (int32_t)U;
  __syncthreads();

  // D. Outputs: the tile table and the unit range and first tile of every
  // workgroup.
  const int64_t alpha = p.split_kv ? p.piece_units : 0;
  const int64_t Uv = U + alpha * M;
  // Ranges used: all p.grid workgroups, or fewer when that would leave each
  // fewer than min_units units (short batches: fewer, longer pieces, fewer
  // partials to merge); the remaining workgroups get empty ranges.
  const int G = p.split_kv ? (int)min((int64_t)p.grid, max((int64_t)1, (Uv + p.min_units - 1) / p.min_units))
                           : p.grid;
  // 32-bit divisions when every product below fits (the usual case).
  const bool small = (Uv + alpha + 2) * (int64_t)G < ((int64_t)1 << 31);
  auto cut = [&](int w) -> int64_t {                   // x(w)
    if (Uv < G) return min((int64_t)w, Uv);
    return small ? (int64_t)((uint32_t)w * (uint32_t)Uv / (uint32_t)G) : ((int64_t)w * Uv) / G;
  };
  auto cnt = [&](int64_t v) -> int {                   // cuts x(w), w in [0, G], below v
    if (v <= 0) return 0;
    if (Uv < G) return v <= Uv ? (int)v : G + 1;
    const int64_t c = small ? (int64_t)(((uint32_t)v * (uint32_t)G + (uint32_t)Uv - 1) / (uint32_t)Uv)
                            : (v * G + Uv - 1) / Uv;
    return (int)min(c, (int64_t)G + 1);
  };
  // The unit range of every workgroup: each tile's thread loops over the
  // workgroups whose cuts land in it, or, when tiles hold many ranges each
  // (short decode batches), each range is found by its own thread.
  const bool per_range = p.split_kv && (int64_t)G > 4 * (int64_t)M;
  for (int i = threadIdx.x; i < M; i += kSchedThreads) {
    const int b = tb[i];
    MTile t;
    t.b = b / p.kvh;
    t.kvg = b - t.b * p.kvh;
    t.row0 = trow[2 * i];
    t.nrows = trow[2 * i + 1];
    t.kv_lo = tkv[2 * i];
    t.kv_hi = tkv[2 * i + 1];
    t.unit0 = u0[i];
    t.tok0 = tlo[b];
    t.past = pst[b];
    if (p.split_kv) {
      const int64_t Vi = u0[i] + alpha * i, Vn = u0[i + 1] + alpha * (i + 1);
      const int Wi = cnt(Vi), Wn = cnt(Vn);
      const int Pi = cnt(Vi + alpha + 1) - Wi;         // cuts inside the virtual prefix
      t.w_first = Wi + Pi - 1;
      t.npieces = Wn - t.w_first;
      t.part_base = Pi > 0 ? t.w_first : p.grid + i;   // slot of the first piece
      if (!per_range) {
        for (int w = Wi; w < Wn; ++w) {
          const int64_t o = cut(w) - Vi - alpha;
          p.wg_range[w] = u0[i] + (int32_t)min(max(o, (int64_t)0), (int64_t)(u0[i + 1] - u0[i]));
          p.wg_tile[w] = i;
        }
      }
    } else {
      t.w_first = i;
      t.npieces = 1;
      t.part_base = -1;
      p.wg_range[i] = u0[i];
      p.wg_tile[i] = i;
    }
    p.mt[i] = t;
  }
  // Workgroups past the last cut inside a tile: empty ranges at the end.
  const int wtail = p.split_kv ? (M > 0 ? cnt(Uv) : 0) : M;
  if (per_range) {
    // Every other range, one workgroup per thread: its cut x(w) falls in the
    // virtual span [V_i, V_i+1) of tile i (V_i = u0[i] + alpha i, found by
    // binary search) and starts at that tile's unit x(w) - V_i - alpha,
    // clamped into the tile's units.
    for (int w = threadIdx.x; w < wtail; w += kSchedThreads) {
      const int64_t x = cut(w);
      int lo = 0, hi = M - 1;                          // last i with V_i <= x (V_0 = 0)
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)u0[mid] + alpha * mid <= x) lo = mid; else hi = mid - 1;
      }
      const int64_t o = x - ((int64_t)u0[lo] + alpha * lo) - alpha;
      p.wg_range[w] = u0[lo] + (int32_t)min(max(o, (int64_t)0), (int64_t)(u0[lo + 1] - u0[lo]));
      p.wg_tile[w] = lo;
    }
  }
  for (int w = wtail + (int)threadIdx.x; w <= p.grid; w += kSchedThreads) {
    p.wg_range[w] = (int32_t)U;
    if (w < p.grid) p.wg_tile[w] = max(M - 1, 0);
  }
  if (threadIdx.x == 0) {
    MTile t = {};
    t.unit0 = (int32_t)U;
    p.mt[M] = t;
    p.header[0] = (int32_t)U;
    p.header[1] = M;
    p.header[2] = G;   // ranges in use (the rest are empty)
  }
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(SchedParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kSchedLdsBytes];
  if (p.wblocks > 0 && (int)blockIdx.x >= p.wblock0) {
    // Write phase of a fused call: it reads none of what the schedule and the
    // query pre-pass produce, and the attention launch that reads the rows it
    // stores follows this launch on the stream.
    const int64_t r = (int64_t)(blockIdx.x - p.wblock0) * (kSchedThreads / 64) + (threadIdx.x >> 6);
    const bool vrow = r >= p.T;                        // separate layout: value rows after the key rows
    const int64_t t = vrow ? r - p.T : r;
    if (t < p.T && (!vrow || p.wval)) {
      const uint16_t* src = vrow ? p.wval : p.wkey;
      uint16_t* dst = vrow ? p.wvcache : p.wcache;
      const int hw = vrow ? p.vhs : p.hs;             // channels per head; RoPE on key rows only
      const int rot = vrow ? 0 : (p.rd > 0);
      if (p.dtype == 16)
        write_row<BF16>(src, p.cos_t, p.sin_t, p.wslot, p.cumseq, p.past, dst, t, p.kvh * hw, hw, p.ro, p.rd,
                        rot, p.interleaved, p.B, p.wslots, p.prow, threadIdx.x & 63);
      else
        write_row<F16>(src, p.cos_t, p.sin_t, p.wslot, p.cumseq, p.past, dst, t, p.kvh * hw, hw, p.ro, p.rd,
                       rot, p.interleaved, p.B, p.wslots, p.prow, threadIdx.x & 63);
    }
    return;
  }
  if (blockIdx.x > 0) {
    // Sequence bounds staged behind the transpose buffer when they fit (one
    // coalesced load per block instead of chains of dependent global loads).
    constexpr int kTBytes = kPreTBytes + kPreRowBytes;   // transpose buffer and row placements
    static_assert(kPreTBytes % 16 == 0 && kTBytes < kSchedLdsBytes, "pre-pass LDS");
    int32_t* const stage = (int32_t*)(lds + kTBytes);
    const bool staged = 2 * (int64_t)p.B + 1 <= (kSchedLdsBytes - kTBytes) / 4;
    if (staged) {
      for (int b = threadIdx.x; b <= p.B; b += kSchedThreads) {
        stage[b] = p.cumseq[b];
        if (b < p.B) stage[p.B + 1 + b] = p.past[b];
      }
      __syncthreads();
    }
    const int32_t* cum = staged ? stage : p.cumseq;
    const int32_t* pst = staged ? stage + p.B + 1 : p.past;
    const int64_t groups = (p.T * p.H + kPreRows - 1) / kPreRows;
    for (int64_t gi = blockIdx.x - 1; gi < groups; gi += p.rope_blocks) {
      if (p.dtype == 16) query_frag_rows<BF16>(p, gi * kPreRows, lds, cum, pst);
      else query_frag_rows<F16>(p, gi * kPreRows, lds, cum, pst);
    }
    return;
  }
  if (sched_ints(p.B * p.kvh, p.max_mtiles, p.grid) <= kSchedLdsInts) schedule_build<true>(p, (int32_t*)lds);
  else schedule_build<false>(p, (int32_t*)lds);
}

// ---------------------------------------------------------------------------
// Instance table
// ---------------------------------------------------------------------------

PA_DECLARE_ATTN_INSTANCE(lat, bf16, 576, 512, 4, 32)
PA_DECLARE_ATTN_INSTANCE(lat, f16, 576, 512, 4, 32)
PA_DECLARE_ATTN_INSTANCE(lat, bf16, 192, 128, 4, 64)
PA_DECLARE_ATTN_INSTANCE(lat, f16, 192, 128, 4, 64)
PA_DECLARE_ATTN_INSTANCE(lat, bf16, 192, 128, 1, 64)
PA_DECLARE_ATTN_INSTANCE(lat, f16, 192, 128, 1, 64)
PA_DECLARE_ATTN_INSTANCE(lat, bf16, 64, 32, 1, 32)
PA_DECLARE_ATTN_INSTANCE(lat, f16, 64, 32, 1, 32)
PA_DECLARE_ATTN_INSTANCE(lat, bf16, 64, 32, 4, 64)
PA_DECLARE_ATTN_INSTANCE(lat, f16, 64, 32, 4, 64)
PA_DECLARE_ATTN_INSTANCE(sep, bf16, 128, 128, 4, 64)
PA_DECLARE_ATTN_INSTANCE(sep, f16, 128, 128, 4, 64)
PA_DECLARE_ATTN_INSTANCE(sep, bf16, 128, 128, 1, 64)
PA_DECLARE_ATTN_INSTANCE(sep, f16, 128, 128, 1, 64)
PA_DECLARE_ATTN_INSTANCE(sep, bf16, 64, 64, 1, 32)
PA_DECLARE_ATTN_INSTANCE(sep, f16, 64, 64, 1, 32)
PA_DECLARE_ATTN_INSTANCE(sep, bf16, 64, 64, 4, 64)
PA_DECLARE_ATTN_INSTANCE(sep, f16, 64, 64, 4, 64)

struct InstanceEntry {
  int dtype, sep, hsp, vhsp, nw, kt;
  AttnLaunchFn launch;
  AttnOccFn occ;
};

#define PA_SEPV_lat 0
#define PA_SEPV_sep 1
#define PA_ENTRY(LAY, DTC, DTN, HSP, VHSP, NW, KT)                                          \
  {DTC, PA_SEPV_##LAY, HSP, VHSP, NW, KT, &PA_ATTN_FN(LAY, DTN, HSP, VHSP, NW, KT, launch), \
   &PA_ATTN_FN(LAY, DTN, HSP, VHSP, NW, KT, occ)}

static const InstanceEntry kInstances[] = {
    PA_ENTRY(lat, 16, bf16, 576, 512, 4, 32), PA_ENTRY(lat, 10, f16, 576, 512, 4, 32),
    PA_ENTRY(lat, 16, bf16, 192, 128, 4, 64), PA_ENTRY(lat, 10, f16, 192, 128, 4, 64),
    PA_ENTRY(lat, 16, bf16, 192, 128, 1, 64), PA_ENTRY(lat, 10, f16, 192, 128, 1, 64),
    PA_ENTRY(lat, 16, bf16, 64, 32, 1, 32),   PA_ENTRY(lat, 10, f16, 64, 32, 1, 32),
    PA_ENTRY(lat, 16, bf16, 64, 32, 4, 64),   PA_ENTRY(lat, 10, f16, 64, 32, 4, 64),
    PA_ENTRY(sep, 16, bf16, 128, 128, 4, 64), PA_ENTRY(sep, 10, f16, 128, 128, 4, 64),
    PA_ENTRY(sep, 16, bf16, 128, 128, 1, 64), PA_ENTRY(sep, 10, f16, 128, 128, 1, 64),
    PA_ENTRY(sep, 16, bf16, 64, 64, 1, 32),   PA_ENTRY(sep, 10, f16, 64, 64, 1, 32),
    PA_ENTRY(sep, 16, bf16, 64, 64, 4, 64),   PA_ENTRY(sep, 10, f16, 64, 64, 4, 64),
};

static const InstanceEntry* find_instance(int dtype, const AttnConfig& c) {
  for (const auto& e : kInstances)
    if (e.dtype == dtype && e.sep == c.sep && e.hsp == c.hsp && e.vhsp == c.vhsp && e.nw == c.nw && e.kt == c.kt)
      return &e;
  return nullptr;
}

// Scheduling charge of a piece of the generic kernel, in KV tiles: the query
// staging and the epilogue take about three 64-key tiles' time on the
// four-wave (prefill) instances, where a workgroup often holds several short
// pieces; the one-wave decode pieces are long and their staging overlaps the
// first tile copies.
// (Build-time tunables for A/B timing; the defaults are the measured best.)
#ifndef PA_GEN_PIECE4
#define PA_GEN_PIECE4 4
#endif
#ifndef PA_MLA_PIECE
#define PA_MLA_PIECE 10
#endif
#ifndef PA_GEN_PIECE1
#define PA_GEN_PIECE1 2
#endif
// Split-KV: fewest (virtual) KV tiles a workgroup's range holds (short batches
// get fewer, longer pieces).
#ifndef PA_MIN_UNITS
#define PA_MIN_UNITS 4
#endif
static int generic_piece_units(int nw) { return nw >= 4 ? PA_GEN_PIECE4 : PA_GEN_PIECE1; }

bool choose_config(const CallGeom& g, AttnConfig* cfg) {
  // Head-size buckets of the compiled instances; smaller sizes run zero-padded.
  cfg->wide = 0;
  cfg->piece_units = 2;
  cfg->sep = g.sep;
  // Query rows per scheduled sequence (per key/value head in the separate layout).
  const int64_t rows_per_seq = g.B > 0 ? (g.T * (g.H / g.kvh)) / g.B : 0;
  if (g.sep) {
    if (g.hs <= 64 && g.vhs <= 64) { cfg->hsp = 64; cfg->vhsp = 64; }
    else if (g.hs <= 128 && g.vhs <= 128) { cfg->hsp = 128; cfg->vhsp = 128; }
    else return false;
    cfg->nw = rows_per_seq >= 96 ? 4 : 1;
    cfg->kt = (cfg->hsp == 64 && cfg->nw == 1) ? 32 : 64;
    cfg->piece_units = generic_piece_units(cfg->nw);
    return find_instance(g.dtype, *cfg) != nullptr;
  }
  if (g.hs <= 64 && g.vhs <= 32) { cfg->hsp = 64; cfg->vhsp = 32; cfg->kt = 32; }
  else if (g.hs <= 192 && g.vhs <= 128) { cfg->hsp = 192; cfg->vhsp = 128; cfg->kt = 64; }
  else if (g.hs <= 576 && g.vhs <= 512) { cfg->hsp = 576; cfg->vhsp = 512; cfg->kt = 32; cfg->wide = 2; cfg->nw = 4; cfg->piece_units = PA_MLA_PIECE; }
  else return false;
  // Four waves (128 rows) when sequences bring many query rows, one wave otherwise.
  if (!cfg->wide) {
    cfg->nw = rows_per_seq >= 96 ? 4 : 1;
    cfg->piece_units = generic_piece_units(cfg->nw);
  }
  if (cfg->hsp == 64 && cfg->nw == 4) cfg->kt = 64;   // staged query rows need 2 tiles >= 32 * nw rows
  return find_instance(g.dtype, *cfg) != nullptr;
}

hipError_t attn_occupancy(const CallGeom& g, const AttnConfig& cfg, int device, int* blocks_per_cu) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, int, int, int, int>, int> cache;
  const auto key = std::make_tuple(device, g.dtype, cfg.sep, cfg.hsp, cfg.vhsp, cfg.nw, cfg.kt);
  {
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(key);
    if (it != cache.end()) { *blocks_per_cu = it->second; return hipSuccess; }
  }
  const InstanceEntry* e = find_instance(g.dtype, cfg);
  if (!e) return hipErrorInvalidValue;
  int n = 0;
  hipError_t err = e->occ(&n);
  if (err != hipSuccess) return err;
  n = std::max(n, 1);
  std::lock_guard<std::mutex> lk(mu);
  cache[key] = n;
  *blocks_per_cu = n;
  return hipSuccess;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

WsLayout plan_workspace(const CallGeom& g, const AttnConfig& cfg, int num_cus, int blocks_per_cu, bool split_kv) {
  WsLayout L{};
  const int RW = cfg.rows();
  // Query tiles: T * H rows over the scheduled sequences (each sequence once per
  // key/value head), at most one partial tile per non-empty scheduled sequence.
  L.max_mtiles = (g.T * g.H + RW - 1) / RW + std::min<int64_t>(g.B, g.T) * g.kvh;
  const int64_t g_split = (int64_t)num_cus * blocks_per_cu;
  L.grid = (int)(split_kv ? g_split : std::max<int64_t>(L.max_mtiles, 1));
  L.ranges = L.grid;
  L.part_cap = split_kv ? L.max_mtiles + L.ranges : 0;
  size_t off = 0;
  L.off_header = off; off = align256(off + 16 * sizeof(int32_t));
  L.off_wg_range = off; off = align256(off + (size_t)(L.ranges + 1) * sizeof(int32_t));
  L.off_wg_tile = off; off = align256(off + (size_t)L.ranges * sizeof(int32_t));
  L.sched_ints = sched_ints(g.B * g.kvh, L.max_mtiles, L.ranges);
  L.off_sched = off; off = align256(off + (size_t)L.sched_ints * sizeof(int32_t));
  L.off_mtiles = off; off = align256(off + (size_t)(L.max_mtiles + 1) * sizeof(MTile));
  L.off_part_ml = off; off = align256(off + (size_t)L.part_cap * RW * 2 * sizeof(float));
  // Partial outputs (bfloat16 for bfloat16 outputs, float32 for float16
  // ones; PartF32 in the kernels): rows padded by 16 bytes and slots by 256
  // bytes so concurrent pieces do not sit at power-of-two strides.
  const int pe = g.dtype == 10 ? 4 : 2;   // partial element bytes
  L.part_row = cfg.vhsp + 16 / pe;
  L.part_slot = (int64_t)RW * L.part_row + 256 / pe;
  L.off_part_o = off; off = align256(off + (size_t)L.part_cap * L.part_slot * pe);
  L.off_qfrag = 0;
  if (cfg.wide == 2) {
    L.off_qfrag = off;
    off = align256(off + (size_t)(g.T * g.H * cfg.hsp) * 2);
  }
  L.total = off;
  return L;
}

hipError_t launch_attention(const CallGeom& g, const AttnConfig& cfg, const WsLayout& ws, bool split_kv,
                            const void* query, const void* cache, const void* value_cache, const void* cos_t,
                            const void* sin_t, const int32_t* cumseq, const int32_t* past,
                            const int32_t* block_table, void* out, void* workspace, hipStream_t stream,
                            const hipEvent_t* ev, const FusedWrite* fw) {
  if (g.T == 0) return hipSuccess;
  const InstanceEntry* e = find_instance(g.dtype, cfg);
  if (!e) return hipErrorInvalidValue;
  uint8_t* wsb = (uint8_t*)workspace;
  SchedParams sp;
  sp.cumseq = cumseq;
  sp.past = past;
  sp.B = g.B;
  sp.max_pos = (int)((int64_t)g.MB * g.bs);
  sp.kvh = g.kvh;
  sp.H = g.H / g.kvh;
  sp.RW = cfg.rows();
  sp.KT = cfg.kt;
  sp.window = g.window;
  sp.grid = ws.ranges;
  sp.split_kv = split_kv ? 1 : 0;
  sp.max_mtiles = ws.max_mtiles;
  sp.part_cap = ws.part_cap;
  sp.header = (int32_t*)(wsb + ws.off_header);
  sp.wg_range = (int32_t*)(wsb + ws.off_wg_range);
  sp.wg_tile = (int32_t*)(wsb + ws.off_wg_tile);
  sp.sched = (int32_t*)(wsb + ws.off_sched);
  sp.piece_units = split_kv ? cfg.piece_units : 0;
  sp.min_units = PA_MIN_UNITS;
  sp.mt = (MTile*)(wsb + ws.off_mtiles);
  sp.query = (const uint16_t*)query;
  sp.cos_t = (const uint16_t*)cos_t;
  sp.sin_t = (const uint16_t*)sin_t;
  sp.qfrag = ws.off_qfrag ? (uint16_t*)(wsb + ws.off_qfrag) : nullptr;
  sp.hsp = cfg.hsp;
  sp.T = g.T;
  sp.prow = g.do_rotary ? g.P : 1;
  sp.hs = g.hs;
  sp.ro = g.ro;
  sp.rd = g.do_rotary ? g.rd : 0;   // 0: no rotary channels
  sp.interleaved = g.interleaved;
  sp.dtype = g.dtype;
  // Query pre-pass blocks: one per kPreRows query rows, at most kPrepassBlocks
  // (four per compute unit of a 256-CU part, as many as the launch's LDS lets
  // a CU hold; grid-stride loop).
  constexpr int64_t kPrepassBlocks = 1024;
  const int64_t rope_groups = sp.qfrag ? (g.T * g.H + kPreRows - 1) / kPreRows : 0;
  const int64_t rope_blocks = std::min<int64_t>(rope_groups, kPrepassBlocks);
  sp.rope_blocks = (int)rope_blocks;
  // Write rows of a fused call: four per block (one per wave), after the
  // pre-pass blocks.
  sp.wkey = fw ? (const uint16_t*)fw->key : nullptr;
  sp.wslot = fw ? fw->slot_mapping : nullptr;
  sp.wcache = fw ? (uint16_t*)fw->key_cache : nullptr;
  sp.wval = fw ? (const uint16_t*)fw->value : nullptr;
  sp.wvcache = fw ? (uint16_t*)fw->value_cache : nullptr;
  sp.vhs = g.vhs;
  sp.wslots = g.NB * g.bs;
  sp.wblock0 = (int)(1 + rope_blocks);
  const int64_t wrows = fw ? (fw->value ? 2 * g.T : g.T) : 0;
  sp.wblocks = (int)((wrows + kSchedThreads / 64 - 1) / (kSchedThreads / 64));
  schedule_kernel<<<(unsigned)(1 + rope_blocks + sp.wblocks), kSchedThreads, 0, stream>>>(sp);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  AttnParams ap;
  ap.query = (const uint16_t*)query;
  ap.cache = (const uint16_t*)cache;
  ap.cos_t = (const uint16_t*)cos_t;
  ap.sin_t = (const uint16_t*)sin_t;
  ap.bt = block_table;
  ap.out = (uint16_t*)out;
  ap.wg_range = sp.wg_range;
  ap.wg_tile = sp.wg_tile;
  ap.mt = sp.mt;
  ap.header = sp.header;
  ap.part_ml = (float*)(wsb + ws.off_part_ml);
  ap.part_o = (void*)(wsb + ws.off_part_o);
  ap.part_slot = ws.part_slot;
  ap.part_row = ws.part_row;
  ap.qfrag = sp.qfrag;
  ap.H = g.H / g.kvh;
  ap.nblk = (int)g.NB;   // NB * block_size <= INT32_MAX (checked by the entry points)
  // Decode-shaped call (no more tokens than sequences, a token's heads within one
  // query tile): each KV row is read by one query tile only, so the four-wave
  // 576/512 kernel's copies take the streaming cache policy.
  ap.kv_stream = (g.T <= g.B && ap.H <= cfg.rows()) ? 1 : 0;
  // More than eight pieces per query tile on average (one query tile per
  // scheduled sequence in such a call).
  ap.many_pieces = (split_kv && ap.kv_stream && ws.grid > 8 * (int64_t)g.B * g.kvh) ? 1 : 0;
  ap.prow = g.do_rotary ? g.P : 1;
  ap.vcache = (const uint16_t*)value_cache;
  ap.Hq = g.H;
  ap.krs = g.kvh * g.hs;
  ap.vrs = g.kvh * g.vhs;
  ap.hs = g.hs;
  ap.vhs = g.vhs;
  ap.bs_log2 = g.bs_log2;
  ap.MB = g.MB;
  ap.ro = g.ro;
  ap.rd = g.rd;
  ap.do_rotary = g.do_rotary;
  ap.interleaved = g.interleaved;
  ap.window = g.window;
  ap.scale = g.scale;
  ap.scale_log2 = g.scale * kLog2e;
  ap.softcap = g.softcap > 0.0f ? g.softcap : 0.0f;
  ap.softcap_inv = g.softcap > 0.0f ? 1.0f / g.softcap : 0.0f;
  return e->launch(ap, ws.grid, split_kv, (int)ws.max_mtiles, stream, ev);
}

}  // namespace pa
