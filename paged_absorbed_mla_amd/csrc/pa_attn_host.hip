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

#include <algorithm>
#include <mutex>
#include <map>
#include <tuple>

namespace pa {

struct SchedParams {
  const int32_t* cumseq;
  const int32_t* past;
  int B, H, RW, KT, window, grid, split_kv;
  int max_pos;       // max_blocks_per_seq * block_size: past lengths are clamped to it
  int piece_units;   // virtual KV tiles charged at the start of every query tile
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
  uint32_t* zero16;
};

constexpr int kSchedThreads = 256;

// Exclusive prefix sum over n values get(i), written with put(i, prefix);
// returns the total. Every thread of the block must call it. Per chunk of
// kSchedThreads values: a shuffle scan inside each wave, then every thread
// adds the totals of the waves before its own (read from LDS in parallel, no
// serial pass).
template <typename Get, typename Put>
__device__ int64_t block_exclusive_scan(int64_t n, Get get, Put put) {
  constexpr int NWV = kSchedThreads / 64;
  __shared__ int64_t wave_sums[NWV];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t carry = 0;
  for (int64_t base = 0; base < n; base += kSchedThreads) {
    const int64_t idx = base + threadIdx.x;
    const int64_t v = idx < n ? get(idx) : 0;
    int64_t x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t y = __shfl_up(x, d);
      if (lane >= d) x += y;
    }
    if (lane == 63) wave_sums[wave] = x;
    __syncthreads();
    int64_t before = 0, total = 0;
#pragma unroll
    for (int k = 0; k < NWV; ++k) {
      const int64_t ws = wave_sums[k];
      before += k < wave ? ws : 0;
      total += ws;
    }
    if (idx < n) put(idx, carry + before + x - v);
    carry += total;
    __syncthreads();
  }
  return carry;
}

// In-place inclusive prefix maximum of a[0, n) (LDS or global); every thread
// of the block must call it.
__device__ void block_inclusive_max_scan(int32_t* a, int64_t n) {
  constexpr int NWV = kSchedThreads / 64;
  __shared__ int32_t wave_max[NWV];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t carry = INT32_MIN;
  for (int64_t base = 0; base < n; base += kSchedThreads) {
    const int64_t idx = base + threadIdx.x;
    int32_t x = idx < n ? a[idx] : INT32_MIN;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t y = __shfl_up(x, d);
      if (lane >= d) x = max(x, y);
    }
    if (lane == 63) wave_max[wave] = x;
    __syncthreads();
    int32_t before = carry, total = carry;
#pragma unroll
    for (int k = 0; k < NWV; ++k) {
      const int32_t wm = wave_max[k];
      if (k < wave) before = max(before, wm);
      total = max(total, wm);
    }
    if (idx < n) a[idx] = max(before, x);
    carry = total;
    __syncthreads();
  }
}

// Workgroup w covers units [wg_range[w], wg_range[w+1]); the one that holds
// unit u is the last w with wg_range[w] <= u.
__device__ __forceinline__ int wg_of_unit(const int32_t* wg_range, int grid, int u) {
  int lo = 0, hi = grid - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (wg_range[mid] <= u) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Blocks 1.. of the schedule launch: the query in the four-wave kernel's
// fragment order, RoPE applied (float32 math, nearest-even rounding; the same
// rotation the write phase applies to key rows). Each sequence's rows are cut
// into blocks of 32 (the rows one wave holds); a block whose first row is R0
// and which has nv rows keeps the span [R0, R0 + nv) * hsp and stores 8-channel
// chunk c of its row l (zero past hs) at chunk c * nv + l, so the wave reads
// k-step s (chunks 2 s and 2 s + 1 of every row) as one contiguous run of
// 32 nv bytes. Threads take chunks in destination order (coalesced stores).
// `cum` and `pst` are cumulative_sequence_length and past_seqlens (staged in
// LDS when they fit).
//
// Where chunk d of the fragment-ordered copy comes from: query row R and
// channel c0 (the chunk's first), and the row's sequence b.
// A chunk whose token the sequence bounds do not place inside [0, T) (only a
// violated precondition does that) gets c0 = hsp: it is stored as zeros and
// nothing is read for it.
struct FragSrc {
  int64_t R;
  int c0, b;
};

__device__ __forceinline__ FragSrc frag_source(const SchedParams& p, int64_t d, const int32_t* cum) {
  const int cpr = p.hsp >> 3;                          // chunks per row
  const int64_t Rg = d / cpr;                          // a row of the block holding chunk d
  const int64_t tok = Rg / p.H;
  FragSrc f;
  f.b = find_seq(cum, p.B, tok);
  const int64_t lo = cum[f.b], hi = cum[f.b + 1];
  if (!(0 <= lo && lo <= tok && tok < hi && hi <= p.T)) {
    f.R = 0;
    f.c0 = p.hsp;
    return f;
  }
  const int64_t s0 = lo * p.H;                         // the sequence's first row
  const int64_t rows_b = (hi - lo) * p.H;
  const int64_t k32 = (Rg - s0) & ~(int64_t)31;        // block's first row within the sequence
  const int64_t R0 = s0 + k32;
  const int nv = (int)min((int64_t)32, rows_b - k32);  // >= 1: Rg lies in the block
  const int local = (int)(d - R0 * cpr);               // in [0, nv * cpr)
  const int c = local / nv;
  f.R = R0 + (local - c * nv);
  f.c0 = c * 8;
  return f;
}

// Chunks d0, d0 + stride, ... (KB of them, those below n) of the copy: the
// plain loads of the batch go out together, then rotary chunks are rotated
// and every chunk is stored.
template <typename DT, int KB>
__device__ __forceinline__ void query_frag_batch(const SchedParams& p, int64_t d0, int64_t stride, int64_t n,
                                                 const int32_t* cum, const int32_t* pst) {
  FragSrc f[KB];
  u32x4_t v[KB];
#pragma unroll
  for (int k = 0; k < KB; ++k) {
    const int64_t d = d0 + k * stride;
    v[k] = u32x4_t{0u, 0u, 0u, 0u};
    if (d < n) {
      f[k] = frag_source(p, d, cum);
      if (f[k].c0 < p.hs) v[k] = *(const u32x4_t*)(p.query + f[k].R * p.hs + f[k].c0);
    }
  }
#pragma unroll
  for (int k = 0; k < KB; ++k) {
    const int64_t d = d0 + k * stride;
    if (d >= n) continue;
    const int c0 = f[k].c0;
    if (p.rd > 0 && c0 >= p.ro && c0 < p.ro + p.rd && c0 < p.hs) {
      const int b = f[k].b;
      float x[8];
      unpack8<DT>(v[k], x);
      const int64_t t = f[k].R / p.H;
      const int64_t pos = min(max((int64_t)pst[b] + (t - (int64_t)cum[b]), (int64_t)0), p.prow - 1);
      rope_chunk<DT>(x, p.query + f[k].R * p.hs, c0, p.ro, p.rd, p.interleaved, pos, p.cos_t, p.sin_t);
      v[k] = pack8<DT>(x);
    }
    *(u32x4_t*)(p.qfrag + d * 8) = v[k];
  }
}

// Block 0 of the schedule launch builds the whole schedule in working arrays
// and writes its outputs (tile table, workgroup ranges, header) only at the
// end: a global store inside the build would make every later barrier wait
// for its write to complete. The arrays live in LDS when they fit (then the
// build runs on LDS instructions: IN_LDS is a template argument, so the
// compiler sees the LDS array itself), else in the workspace.
constexpr int kSchedLdsInts = 12288;

__host__ __device__ inline int64_t sched_ints(int B, int64_t max_mtiles, int grid) {
  return 3 * (int64_t)B + 2 + 9 * max_mtiles + 1 + 2 * (int64_t)grid + 1;
}

template <bool IN_LDS>
__device__ __forceinline__ void schedule_build(const SchedParams& p, int32_t* lds_arr) {
  int32_t* const base = IN_LDS ? lds_arr : p.sched;
  int32_t* const cum = base;                           // [B + 1] cumulative_sequence_length
  int32_t* const pst = cum + (p.B + 1);                // [B] past lengths (negative -> 0)
  int32_t* const sbase = pst + p.B;                    // [B + 1] first query tile of each sequence
  int32_t* const u0 = sbase + (p.B + 1);               // [max_mtiles + 1] KV tiles, then first unit
  int32_t* const np = u0 + (p.max_mtiles + 1);        // [max_mtiles] workgroups per query tile
  int32_t* const tb = np + p.max_mtiles;               // [max_mtiles] sequence of each tile
  int32_t* const trow = tb + p.max_mtiles;             // [max_mtiles] first row, then rows (2 x)
  int32_t* const tkv = trow + 2 * p.max_mtiles;        // [max_mtiles] kv_lo, kv_hi (2 x)
  int32_t* const wr = tkv + 2 * p.max_mtiles;          // [grid + 1] unit range of every workgroup
  int32_t* const wt = wr + (p.grid + 1);               // [grid] query tile of every workgroup
  int32_t* const tw0 = wt + p.grid;                    // [max_mtiles] first workgroup of each tile
  int32_t* const tw1 = tw0 + p.max_mtiles;             // [max_mtiles] last workgroup of each tile

  // Sequence bounds and past lengths, forced into the ranges the
  // preconditions promise (a violated precondition then gives unspecified
  // values but no access outside the caller's buffers): bounds clamped into
  // [0, T] and made non-decreasing, past lengths into [0, MB * bs].
  for (int b = threadIdx.x; b <= p.B; b += kSchedThreads) {
    cum[b] = (int32_t)min(max((int64_t)p.cumseq[b], (int64_t)0), p.T);
    if (b < p.B) pst[b] = min(max(p.past[b], 0), p.max_pos);
  }
  __syncthreads();
  block_inclusive_max_scan(cum, p.B + 1);
  // A. query tiles per sequence, prefix-summed into sbase.
  const int64_t M_all = block_exclusive_scan(
      p.B,
      [&](int64_t b) -> int64_t {
        const int64_t rows = (int64_t)(cum[b + 1] - cum[b]) * p.H;
        return (rows + p.RW - 1) / p.RW;
      },
      [&](int64_t b, int64_t v) { sbase[b] = (int32_t)v; });
  // M cannot exceed max_mtiles when cumseq[B] = T (a precondition); clamp so a
  // violated precondition cannot write past the tile table.
  const int M = (int)min(M_all, p.max_mtiles);
  if (threadIdx.x == 0) sbase[p.B] = (int32_t)M_all;
  __syncthreads();
  // B. describe every query tile; its KV tile count goes to u0 for now.
  for (int i = threadIdx.x; i < M; i += kSchedThreads) {
    int lo = 0, hi = p.B - 1;  // last b with sbase[b] <= i
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sbase[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int rows = (cum[b + 1] - cum[b]) * p.H;
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
  // C. units: prefix sum of KV tiles.
  const int64_t U = block_exclusive_scan(
      M, [&](int64_t i) -> int64_t { return u0[i]; }, [&](int64_t i, int64_t v) { u0[i] = (int32_t)v; });
  if (threadIdx.x == 0) u0[M] = (int32_t)U;
  __syncthreads();
  // D. unit range of every workgroup. Split-KV: the units are laid out with
  // piece_units virtual units before each query tile (the cost of the query
  // load and epilogue a piece adds), and the virtual line is cut evenly; a
  // workgroup that enters a second query tile thus takes fewer KV tiles. A
  // cut inside a tile's virtual prefix falls on the tile's first unit.
  // Empty ranges sit only at the end or right before a tile's first
  // workgroup, so the workgroups that share a query tile are consecutive and
  // each of them writes its partial slot.
  const int64_t alpha = p.piece_units;
  const int64_t Uv = U + alpha * M;
  // Cut x(w) = floor(w Uv / grid) as w q + floor(w r / grid) with Uv = q grid
  // + r: one 64-bit division per thread instead of one per workgroup
  // (w r < grid^2 fits 32 bits for grids below 65536, the split launches'
  // compute-unit multiples).
  const int64_t vq = Uv / p.grid;
  const uint32_t vr = (uint32_t)(Uv - vq * p.grid);
  for (int w = threadIdx.x; w <= p.grid; w += kSchedThreads) {
    int32_t v;
    if (!p.split_kv) {
      v = u0[min(w, M)];
    } else if (M == 0) {
      v = 0;
    } else {
      const int64_t x = Uv < p.grid ? min((int64_t)w, Uv)
                        : p.grid < 65536 ? (int64_t)w * vq + (int64_t)(((uint32_t)w * vr) / (uint32_t)p.grid)
                                         : ((int64_t)w * Uv) / p.grid;
      int lo = 0, hi = M - 1;   // last tile whose virtual start is <= x
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (u0[mid] + alpha * mid <= x) lo = mid; else hi = mid - 1;
      }
      const int64_t o = x - (u0[lo] + alpha * lo);
      v = (int32_t)min(u0[lo] + max(o - alpha, (int64_t)0), (int64_t)u0[lo + 1]);
    }
    wr[w] = v;
  }
  __syncthreads();
  // E. pieces per query tile, and the query tile holding each workgroup's
  // first unit (the last i with u0[i] <= wr[w]).
  for (int i = threadIdx.x; i < M; i += kSchedThreads) {
    const int w0 = wg_of_unit(wr, p.grid, u0[i]);
    const int w1 = wg_of_unit(wr, p.grid, u0[i + 1] - 1);
    np[i] = w1 - w0 + 1;
    tw0[i] = w0;
    tw1[i] = w1;
  }
  for (int w = threadIdx.x; w < p.grid; w += kSchedThreads) {
    const int uw = wr[w];
    int lo = 0, hi = M > 0 ? M - 1 : 0;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (u0[mid] <= uw) lo = mid; else hi = mid - 1;
    }
    wt[w] = lo;
  }
  __syncthreads();
  // F. partial slots for the tiles that several workgroups share; np[i]
  // becomes the tile's first slot (-1: one workgroup, no partial results).
  const int64_t slots = block_exclusive_scan(
      M, [&](int64_t i) -> int64_t { const int n = np[i]; return n > 1 ? n : 0; },
      [&](int64_t i, int64_t v) { np[i] = np[i] > 1 ? (int32_t)v : -1; });
  __syncthreads();
  // Outputs, all stores at the end.
  if (threadIdx.x < 4) p.zero16[threadIdx.x] = 0u;
  for (int i = threadIdx.x; i < M; i += kSchedThreads) {
    MTile t;
    t.b = tb[i];
    t.row0 = trow[2 * i];
    t.nrows = trow[2 * i + 1];
    t.kv_lo = tkv[2 * i];
    t.kv_hi = tkv[2 * i + 1];
    t.unit0 = u0[i];
    t.w_first = tw0[i];
    t.npieces = tw1[i] - tw0[i] + 1;
    t.part_base = np[i];
    t.tok0 = cum[t.b];
    t.past = pst[t.b];
    t.pad = 0;
    p.mt[i] = t;
  }
  if (threadIdx.x == 0) {
    MTile t = {};
    t.unit0 = (int32_t)U;
    p.mt[M] = t;
    p.header[0] = (int32_t)U;
    p.header[1] = M;
    p.header[2] = (int32_t)slots;
  }
  for (int w = threadIdx.x; w <= p.grid; w += kSchedThreads) {
    p.wg_range[w] = wr[w];
    if (w < p.grid) p.wg_tile[w] = wt[w];
  }
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(SchedParams p) {
  __shared__ int32_t lds_arr[kSchedLdsInts];
  if (blockIdx.x > 0) {
    // Token -> sequence search over LDS copies of the sequence bounds (one
    // coalesced load per block instead of a chain of dependent global loads).
    const bool staged = 2 * p.B + 1 <= kSchedLdsInts;
    if (staged) {
      for (int b = threadIdx.x; b <= p.B; b += kSchedThreads) {
        lds_arr[b] = p.cumseq[b];
        if (b < p.B) lds_arr[p.B + 1 + b] = p.past[b];
      }
      __syncthreads();
    }
    const int32_t* cum = staged ? lds_arr : p.cumseq;
    const int32_t* pst = staged ? lds_arr + p.B + 1 : p.past;
    // Grid-stride over the chunks: the launch holds few of these blocks (the
    // LDS array sized for block 0 allows three per CU), each thread taking a
    // chunk per stride.
    constexpr int KB = 4;   // chunks per thread whose loads are in flight together
    const int64_t n = p.T * p.H * (p.hsp >> 3);
    const int64_t stride = (int64_t)(gridDim.x - 1) * kSchedThreads;
    for (int64_t idx = (int64_t)(blockIdx.x - 1) * kSchedThreads + threadIdx.x; idx < n; idx += KB * stride) {
      if (p.dtype == 16) query_frag_batch<BF16, KB>(p, idx, stride, n, cum, pst);
      else query_frag_batch<F16, KB>(p, idx, stride, n, cum, pst);
    }
    return;
  }
  if (sched_ints(p.B, p.max_mtiles, p.grid) <= kSchedLdsInts) schedule_build<true>(p, lds_arr);
  else schedule_build<false>(p, lds_arr);
}

// ---------------------------------------------------------------------------
// Instance table
// ---------------------------------------------------------------------------

PA_DECLARE_ATTN_INSTANCE(bf16, 576, 512, 4, 32)
PA_DECLARE_ATTN_INSTANCE(f16, 576, 512, 4, 32)
PA_DECLARE_ATTN_INSTANCE(bf16, 192, 128, 4, 64)
PA_DECLARE_ATTN_INSTANCE(f16, 192, 128, 4, 64)
PA_DECLARE_ATTN_INSTANCE(bf16, 192, 128, 1, 64)
PA_DECLARE_ATTN_INSTANCE(f16, 192, 128, 1, 64)
PA_DECLARE_ATTN_INSTANCE(bf16, 64, 32, 1, 32)
PA_DECLARE_ATTN_INSTANCE(f16, 64, 32, 1, 32)
PA_DECLARE_ATTN_INSTANCE(bf16, 64, 32, 4, 64)
PA_DECLARE_ATTN_INSTANCE(f16, 64, 32, 4, 64)

struct InstanceEntry {
  int dtype, hsp, vhsp, nw, kt;
  AttnLaunchFn launch;
  AttnOccFn occ;
};

#define PA_ENTRY(DTC, DTN, HSP, VHSP, NW, KT)                                               \
  {DTC, HSP, VHSP, NW, KT, &PA_ATTN_FN(DTN, HSP, VHSP, NW, KT, launch),                     \
   &PA_ATTN_FN(DTN, HSP, VHSP, NW, KT, occ)}

static const InstanceEntry kInstances[] = {
    PA_ENTRY(16, bf16, 576, 512, 4, 32),  PA_ENTRY(10, f16, 576, 512, 4, 32),
    PA_ENTRY(16, bf16, 192, 128, 4, 64), PA_ENTRY(10, f16, 192, 128, 4, 64),
    PA_ENTRY(16, bf16, 192, 128, 1, 64), PA_ENTRY(10, f16, 192, 128, 1, 64),
    PA_ENTRY(16, bf16, 64, 32, 1, 32),   PA_ENTRY(10, f16, 64, 32, 1, 32),
    PA_ENTRY(16, bf16, 64, 32, 4, 64),   PA_ENTRY(10, f16, 64, 32, 4, 64),
};

static const InstanceEntry* find_instance(int dtype, const AttnConfig& c) {
  for (const auto& e : kInstances)
    if (e.dtype == dtype && e.hsp == c.hsp && e.vhsp == c.vhsp && e.nw == c.nw && e.kt == c.kt) return &e;
  return nullptr;
}

bool choose_config(const CallGeom& g, AttnConfig* cfg) {
  // Head-size buckets of the compiled instances; smaller sizes run zero-padded.
  cfg->wide = 0;
  cfg->piece_units = 2;
  if (g.hs <= 64 && g.vhs <= 32) { cfg->hsp = 64; cfg->vhsp = 32; cfg->kt = 32; }
  else if (g.hs <= 192 && g.vhs <= 128) { cfg->hsp = 192; cfg->vhsp = 128; cfg->kt = 64; }
  else if (g.hs <= 576 && g.vhs <= 512) { cfg->hsp = 576; cfg->vhsp = 512; cfg->kt = 32; cfg->wide = 2; cfg->nw = 4; cfg->piece_units = 10; }
  else return false;
  // Four waves (128 rows) when sequences bring many query rows, one wave otherwise.
  const int64_t rows_per_seq = g.B > 0 ? (g.T * g.H) / g.B : 0;
  if (!cfg->wide) cfg->nw = rows_per_seq >= 96 ? 4 : 1;
  if (cfg->hsp == 64 && cfg->nw == 4) cfg->kt = 64;   // staged query rows need 2 tiles >= 32 * nw rows
  return find_instance(g.dtype, *cfg) != nullptr;
}

hipError_t attn_occupancy(const CallGeom& g, const AttnConfig& cfg, int device, int* blocks_per_cu) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, int, int, int>, int> cache;
  const auto key = std::make_tuple(device, g.dtype, cfg.hsp, cfg.vhsp, cfg.nw, cfg.kt);
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
  L.max_mtiles = (g.T * g.H + RW - 1) / RW + std::min<int64_t>(g.B, g.T);
  const int64_t g_split = (int64_t)num_cus * blocks_per_cu;
  L.grid = (int)(split_kv ? g_split : std::max<int64_t>(L.max_mtiles, 1));
  L.ranges = L.grid;
  L.part_cap = split_kv ? L.max_mtiles + L.ranges : 0;
  size_t off = 0;
  L.off_header = off; off = align256(off + 16 * sizeof(int32_t));
  L.off_zero = off; off = align256(off + 16);
  L.off_wg_range = off; off = align256(off + (size_t)(L.ranges + 1) * sizeof(int32_t));
  L.off_wg_tile = off; off = align256(off + (size_t)L.ranges * sizeof(int32_t));
  L.sched_ints = sched_ints(g.B, L.max_mtiles, L.ranges);
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
                            const void* query, const void* cache, const void* cos_t, const void* sin_t,
                            const int32_t* cumseq, const int32_t* past, const int32_t* block_table, void* out,
                            void* workspace, hipStream_t stream, const hipEvent_t* ev) {
  if (g.T == 0) return hipSuccess;
  const InstanceEntry* e = find_instance(g.dtype, cfg);
  if (!e) return hipErrorInvalidValue;
  uint8_t* wsb = (uint8_t*)workspace;
  SchedParams sp;
  sp.cumseq = cumseq;
  sp.past = past;
  sp.B = g.B;
  sp.max_pos = (int)((int64_t)g.MB * g.bs);
  sp.H = g.H;
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
  sp.mt = (MTile*)(wsb + ws.off_mtiles);
  sp.zero16 = (uint32_t*)(wsb + ws.off_zero);
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
  // Query pre-pass blocks: at most kPrepassBlocks (two per compute unit of a
  // 256-CU part; grid-stride loop).
  constexpr int64_t kPrepassBlocks = 512;
  const int64_t rope_chunks = sp.qfrag ? g.T * g.H * (cfg.hsp >> 3) : 0;
  const int64_t rope_blocks = std::min<int64_t>((rope_chunks + kSchedThreads - 1) / kSchedThreads, kPrepassBlocks);
  schedule_kernel<<<(unsigned)(1 + rope_blocks), kSchedThreads, 0, stream>>>(sp);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  AttnParams ap;
  ap.query = (const uint16_t*)query;
  ap.cache = (const uint16_t*)cache;
  ap.cos_t = (const uint16_t*)cos_t;
  ap.sin_t = (const uint16_t*)sin_t;
  ap.bt = block_table;
  ap.out = (uint16_t*)out;
  ap.header = sp.header;
  ap.wg_range = sp.wg_range;
  ap.wg_tile = sp.wg_tile;
  ap.mt = sp.mt;
  ap.zero16 = (const uint16_t*)sp.zero16;
  ap.part_ml = (float*)(wsb + ws.off_part_ml);
  ap.part_o = (void*)(wsb + ws.off_part_o);
  ap.part_slot = ws.part_slot;
  ap.part_row = ws.part_row;
  ap.qfrag = sp.qfrag;
  ap.nblk = g.NB;
  ap.prow = g.do_rotary ? g.P : 1;
  ap.H = g.H;
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
