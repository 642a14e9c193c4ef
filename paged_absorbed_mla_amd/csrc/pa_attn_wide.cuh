// Read phase for wide latent rows (head sizes up to 576 / value sizes up to
// 512) on gfx950.
//
// Semantics are those of attn_kernel (pa_attn.cuh): docs.rs page
// "onnx-runtime-ep-cuda src/kernels/paged_attention.rs", "LATENT semantics",
// read phase (device function attn_impl).
//
// Design. One workgroup of eight waves (two per SIMD) owns a 128-row query tile
// (row = token_in_sequence * H + head) and walks a contiguous range of 32-key KV
// tiles, each copied once from the paged cache into LDS:
//   * QK^T is split by rows: wave w computes S^T = K Q^T for rows
//     [16 w, 16 w + 16) on v_mfma_f32_16x16x32 (A = 16 keys x 32 channels read
//     from LDS, B = the wave's 16 RoPE'd query rows, kept in registers), then
//     the online-softmax update for those rows. Its probabilities go to LDS as
//     bf16/f16 P^T fragments, one 16-byte write per lane.
//   * PV is split by value channels: wave w computes O^T = V^T P^T for channels
//     [64 w, 64 w + 64) of all 128 rows (A = V^T from ds_read_b64_tr_b16
//     transposing reads, B = P^T fragments from LDS). Every value byte of a
//     tile is read from LDS once per workgroup, and the per-wave state stays
//     at 72 (query) + 128 (output) registers, so two waves fit per SIMD: a
//     single wave per SIMD cannot issue LDS reads fast enough for this path.
//   * The key order inside a 32-key PV step is permuted consistently: k-index
//     8 g + e of lane group g holds key 4 g + (e & 3) + 16 (e >> 2). These are
//     exactly the keys the QK accumulator lane holds, so P^T is written as-is,
//     and the two transposing reads of a V^T fragment are 16 rows apart (same
//     swizzle, immediate offset).
//   * Running-max corrections travel with P: a wave whose rows moved their
//     reference maximum sets a flag and publishes the per-row factors; PV waves
//     rescale only the row blocks that were flagged.
//   * Copies: NB LDS buffers, up to NB - 1 tiles in flight. Wave w copies keys
//     [4 w, 4 w + 4) of each tile (one cache block, one scalar block-table
//     read), as direct global->LDS loads.
// Two barriers per tile: the first publishes the tile's copies and frees the
// buffer and P area of the previous tile, the second publishes P.
#pragma once

#include "pa_attn.cuh"

namespace pa {

template <typename DT, int HSP, int VHSP, int KT, int NB>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void attn_wide_kernel(AttnParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NW = 8;
  constexpr int RW = 128;                 // rows of a query tile
  constexpr int CPR = HSP / 8;            // 16-byte chunks per LDS row
  constexpr int NKK = HSP / 32;           // QK channel steps
  constexpr int VC = VHSP / NW;           // value channels per wave
  constexpr int NVB = VC / 16;            // 16-channel O^T blocks per row block
  constexpr int NRB = RW / 16;            // 16-row blocks
  constexpr int KW = KT / NW;             // keys each wave copies per tile
  constexpr int SLOTS = KW * CPR;         // 16-byte copies per wave per tile
  constexpr int LOADS = (SLOTS + 63) / 64;
  constexpr int LAST = SLOTS - (LOADS - 1) * 64;   // active lanes of the last copy instruction
  constexpr int BUF_BYTES = KT * CPR * 16;
  constexpr int OFF_P = NB * BUF_BYTES;            // P^T fragments: [row block][lane] x 16 bytes
  constexpr int OFF_CORR = OFF_P + RW * KT * 2;    // [RW] float running-max corrections
  constexpr int OFF_FLAG = OFF_CORR + RW * 4;      // [NW] int: row block rescaled this tile
  constexpr int OFF_L = OFF_FLAG + NW * 4;         // [RW] float softmax denominators
  constexpr int LDS_BYTES = OFF_L + RW * 4;
  constexpr int ROW16 = 16 * CPR * 16;             // 16 LDS rows
  static_assert(KT == 32, "one 32-key PV step per tile");
  static_assert(HSP % 64 == 0 && VC % 16 == 0 && VHSP <= HSP, "head sizes");
  static_assert(KW >= 1 && KW <= 16 && LAST > 0, "copy slice");
  static_assert(NB >= 2 && (NB - 2) * LOADS <= 63, "vmcnt range");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(ROW16 + (NKK / 2) * 128 < 65536, "ds offset range");
  __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[LDS_BYTES];

  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;

  int u = ld_uniform(p.wg_range + blockIdx.x);
  const int u_end = ld_uniform(p.wg_range + blockIdx.x + 1);
  if (u >= u_end) return;
  int i;
  {
    int lo = 0, hi_ = ld_uniform(p.header + 1) - 1;
    while (lo < hi_) {
      const int mid = (lo + hi_ + 1) >> 1;
      if (ld_uniform(&p.mt[mid].unit0) <= u) lo = mid; else hi_ = mid - 1;
    }
    i = lo;
  }
  const bool softcap_on = p.softcap > 0.0f;

  // Copy slot sl = it * 64 + lane of this wave holds chunk (sl % CPR) of key
  // w * KW + sl / CPR at swizzled position. Its source is byte off(it) of the
  // wave's KW cache rows (tile-independent, < 2^16), two offsets per register;
  // chunks at channels >= hs get 0xFFFF, past the buffer descriptor's range
  // (KW * hs * 2 bytes), which reads as zeros.
  constexpr int NOFF = (LOADS + 1) / 2;
  static_assert(KW * HSP * 2 + 16 <= 0xFFFF, "16-bit copy offsets");
  uint32_t load_off2[NOFF];
#pragma unroll
  for (int k2 = 0; k2 < NOFF; ++k2) load_off2[k2] = 0xFFFFFFFFu;
#pragma unroll
  for (int it = 0; it < LOADS; ++it) {
    const int sl = it * 64 + lane;
    const int k = sl / CPR;
    const int lc = (sl - k * CPR) ^ lds_swizzle(w * KW + k);
    const uint32_t off = lc * 8 < p.hs ? (uint32_t)((k * p.hs + lc * 8) * 2) : 0xFFFFu;
    const int sh = (it & 1) * 16;
    load_off2[it >> 1] = (load_off2[it >> 1] & ~(0xFFFFu << sh)) | (off << sh);
  }

  // LDS byte addresses (buffer 0) of this lane's fragment reads.
  // K (QK A operand): key l16 (+16 sub), chunk 4 kk + q4; kk parity selects the base.
  const int swk = lds_swizzle(l16);
  int koff[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) koff[r] = l16 * CPR * 16 + (((4 * r + q4) ^ swk) << 4);
  // V^T (PV A operand), transposing read: lane (g = q4, j = l16 >> 2, q = l16 & 3)
  // points at key 4 g + j (+16), channels VC w + 16 vb + 4 q .. + 3, i.e. chunk
  // 8 (VC w / 8 + ...) with low bits (2 vb + (q >> 1)) ^ swizzle = 2 vb ^ vx.
  const int kr = 4 * q4 + (l16 >> 2);
  const int vx = ((l16 & 3) >> 1) ^ lds_swizzle(kr);
  static_assert(VC % 64 == 0 && NVB <= 4, "a wave's value channels span whole swizzle groups");
  const uint32_t vbase = lds_addr(lds_raw) + kr * CPR * 16 + (VC * w / 8) * 16 + (l16 & 1) * 8;
  auto vaddr = [&](int vb) -> uint32_t { return vbase + (((2 * vb) ^ vx) << 4); };
  const uint32_t paddr = lds_addr(lds_raw) + OFF_P + lane * 16;     // + 1024 * row block
  float* const corr_lds = (float*)(lds_raw + OFF_CORR);
  int* const flag_lds = (int*)(lds_raw + OFF_FLAG);
  float* const l_lds = (float*)(lds_raw + OFF_L);

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
    const int nrb = (t.nrows + 15) >> 4;                 // row blocks holding rows of the tile

    // This lane's QK row.
    const int rq = 16 * w + l16;
    const bool row_ok = rq < t.nrows;
    const int Rq = t.row0 + rq;
    const int tq = Rq / p.H;
    const int pos = row_ok ? past_b + tq : -1;
    const int lo_row = p.window >= 0 ? max(0, pos - p.window) : 0;
    const bool qk_active = 16 * w < t.nrows;

    // Query fragments: this wave's 16 rows are staged in LDS (tile buffers and
    // P area are free between pieces), RoPE'd there in float32 with one lane per
    // rotary pair and rounded to the storage type, then read as B fragments
    // (row l16, channels 32 kk + 8 q4 .. + 8).
    u32x4_t qf[NKK];
    {
      constexpr int QSTRIDE = HSP + 8;                 // elements; padded against bank conflicts
      static_assert(NW * 16 * QSTRIDE * 2 <= OFF_L, "query staging stays clear of the denominators");
      uint16_t* qs = (uint16_t*)lds_raw + w * 16 * QSTRIDE;
      const int lane_s = opaque_lane();
      for (int idx = lane_s; idx < 16 * CPR; idx += 64) {
        const int r = idx / CPR;
        const int c0 = (idx - r * CPR) * 8;
        const int rl = 16 * w + r;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (rl < t.nrows && c0 < p.hs) {
          const int Rr = t.row0 + rl;
          const int tr = Rr / p.H;
          v = *(const u32x4_t*)(p.query + ((int64_t)(cum_b + tr) * p.H + (Rr - tr * p.H)) * p.hs + c0);
        }
        *(u32x4_t*)(qs + r * QSTRIDE + c0) = v;
      }
      if (p.do_rotary) {
        const int hr = p.rd >> 1;
        for (int idx = lane_s; idx < 16 * hr; idx += 64) {
          const int r = idx / hr;
          const int k = idx - r * hr;
          const int rl = 16 * w + r;
          if (rl >= t.nrows) continue;
          const int posr = past_b + (t.row0 + rl) / p.H;
          const int d1 = p.interleaved ? p.ro + 2 * k : p.ro + k;
          const int d2 = p.interleaved ? d1 + 1 : d1 + hr;
          const int64_t pr = min(max((int64_t)posr, (int64_t)0), p.prow - 1);
          const float c = DT::to_f32(p.cos_t[pr * hr + k]);
          const float sn = DT::to_f32(p.sin_t[pr * hr + k]);
          const float x1 = DT::to_f32(qs[r * QSTRIDE + d1]);
          const float x2 = DT::to_f32(qs[r * QSTRIDE + d2]);
          qs[r * QSTRIDE + d1] = (uint16_t)DT::from_f32(x1 * c - x2 * sn);
          qs[r * QSTRIDE + d2] = (uint16_t)DT::from_f32(x2 * c + x1 * sn);
        }
      }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) qf[kk] = *(const u32x4_t*)(qs + (lane_s & 15) * QSTRIDE + 32 * kk + 8 * (lane_s >> 4));
      __syncthreads();   // staging area is reused by the tile buffers
    }
    f32x4_t o[NVB][NRB];
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) o[vb][rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;

    // Exactly LOADS copy instructions per wave per call (vmcnt counts them).
    // The buffer descriptor spans the wave's KW cache rows of the tile; slots of
    // keys outside [kv_lo, kv_hi) use an out-of-range offset and copy zeros.
    auto issue = [&](int tile, int bufi) {
      const int kw0 = tile * KT + w * KW;
      const int blk = clamp_block(ld_uniform(p.bt + (int64_t)b * p.MB + min(kw0 >> p.bs_log2, p.MB - 1)), p.nblk);
      const uint16_t* rows = p.cache + (((int64_t)blk << p.bs_log2) + (kw0 & ((1 << p.bs_log2) - 1))) * p.hs;
      const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(rows, (uint32_t)(KW * p.hs * 2));
      uint8_t* dst0 = lds_raw + bufi * BUF_BYTES + w * SLOTS * 16;
      // Offsets are unpacked here, from opaque copies, so the unpacked values
      // are not hoisted out of the tile loop and kept live across it.
      const int lane_i = opaque_lane();
      uint32_t offs2[NOFF];
#pragma unroll
      for (int k2 = 0; k2 < NOFF; ++k2) {
        offs2[k2] = load_off2[k2];
        asm volatile("" : "+v"(offs2[k2]));
      }
      auto load_off = [&](int it) -> uint32_t { return (offs2[it >> 1] >> ((it & 1) * 16)) & 0xFFFFu; };
      if (kw0 >= t.kv_lo && kw0 + KW <= t.kv_hi) {
#pragma unroll
        for (int it = 0; it < LOADS; ++it)
          if (it < LOADS - 1 || lane_i < LAST)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(dst0 + it * 64 * 16), 16, load_off(it), 0, 0, 0);
      } else {
#pragma unroll
        for (int it = 0; it < LOADS; ++it) {
          if (it < LOADS - 1 || lane_i < LAST) {
            const int j = kw0 + (it * 64 + lane_i) / CPR;
            const uint32_t off = (j >= t.kv_lo && j < t.kv_hi) ? load_off(it) : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(dst0 + it * 64 * 16), 16, off, 0, 0, 0);
          }
        }
      }
    };

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // previous piece's stores
#pragma unroll
    for (int k = 0; k < NB - 1; ++k)
      if (tile_a + k < tile_b) issue(tile_a + k, k);

    for (int tt = tile_a; tt < tile_b; ++tt) {
      const int bufi = (tt - tile_a) % NB;
      const uint32_t boff = (uint32_t)(bufi * BUF_BYTES);
      const int ahead = min(NB - 2, tile_b - 1 - tt);
      vm_wait_tiles<LOADS, NB - 2>(ahead);
      lds_barrier();     // tile tt visible; every wave is done with tile tt - 1 and its P
      if (tt + NB - 1 < tile_b) issue(tt + NB - 1, (tt + NB - 1 - tile_a) % NB);

      // ---- S^T = K Q^T for rows [16 w, 16 w + 16), softmax update, P^T to LDS ----
      const int lane_t = opaque_lane();
      const int l16t = lane_t & 15, q4t = lane_t >> 4;
      if (qk_active) {
        const int key0 = tt * KT;
        constexpr int QPF = 4;
        constexpr int QSTEPS = 2 * NKK;   // step n: channel step n / 2, key half n % 2
        f32x4_t s[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
        const uint8_t* kb0 = lds_raw + boff + koff[0];
        const uint8_t* kb1 = lds_raw + boff + koff[1];
        auto k_frag = [&](int n) -> u32x4_t {
          const int kk = n >> 1, sub = n & 1;
          return *(const u32x4_t*)(((kk & 1) ? kb1 : kb0) + sub * ROW16 + (kk >> 1) * 128);
        };
        u32x4_t ka[QPF];
#pragma unroll
        for (int n = 0; n < QPF; ++n) ka[n] = k_frag(n);
#pragma unroll
        for (int n = 0; n < QSTEPS; ++n) {
          const u32x4_t cur = ka[n % QPF];
          if (n + QPF < QSTEPS) ka[n % QPF] = k_frag(n + QPF);
          s[n & 1] = DT::mfma16(cur, qf[n >> 1], s[n & 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
        // Lane holds keys 16 sub + 4 q4 + e of its row.
        if (softcap_on) {
#pragma unroll
          for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int e = 0; e < 4; ++e) s[sub][e] = softcap_log2(s[sub][e], p.scale, p.softcap, p.softcap_inv);
        } else {
          s[0] *= p.scale_log2;
          s[1] *= p.scale_log2;
        }
        float tmax = -INFINITY;
        if (__all(key0 >= lo_row && key0 + KT - 1 <= pos)) {
#pragma unroll
          for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, s[sub][e]);
        } else {
#pragma unroll
          for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int j = key0 + 16 * sub + 4 * q4t + e;
              const float v = (j <= pos && j >= lo_row) ? s[sub][e] : -INFINITY;
              s[sub][e] = v;
              tmax = fmaxf(tmax, v);
            }
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        // Lazy rescale: the reference max moves only when the tile max exceeds it
        // by more than 8 (log2 units); probabilities stay <= 2^8 and numerator and
        // denominator share the reference, so the result is unchanged.
        const bool bump = tmax > m_run + 8.0f;
        const float m_new = bump ? tmax : m_run;
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float corr = fast_exp2(m_run - m_use);
        const bool rescale = bump && (m_run != -INFINITY);
        m_run = m_new;
        float pv[8];
        float psum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = fast_exp2(s[e >> 2][e & 3] - m_use);
          psum += pv[e];
        }
        l_run = l_run * corr + psum;
        *(u32x4_t*)(lds_raw + OFF_P + w * 1024 + lane_t * 16) = pack8<DT>(pv);
        const bool any_rescale = __any(rescale);
        if (any_rescale && q4t == 0) corr_lds[16 * w + l16t] = corr;
        if (lane_t == 0) flag_lds[w] = any_rescale ? 1 : 0;
      }
      lds_barrier();     // P^T, corrections and flags of tile tt visible

      // ---- O^T += V^T P^T for channels [VC w, VC w + VC) of all rows ----
      {
        const u32x4_t fl0 = *(const u32x4_t*)(flag_lds);
        const u32x4_t fl1 = *(const u32x4_t*)(flag_lds + 4);
        const int flags = __builtin_amdgcn_readfirstlane((int)((fl0[0] != 0u) | ((fl0[1] != 0u) << 1) |
                                                               ((fl0[2] != 0u) << 2) | ((fl0[3] != 0u) << 3) |
                                                               ((fl1[0] != 0u) << 4) | ((fl1[1] != 0u) << 5) |
                                                               ((fl1[2] != 0u) << 6) | ((fl1[3] != 0u) << 7)));
        const int live = flags & ((1 << nrb) - 1);
        if (live) {
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) {
            if (live & (1 << rb)) {
              const float c = corr_lds[16 * rb + l16t];
#pragma unroll
              for (int vb = 0; vb < NVB; ++vb) o[vb][rb] *= c;
            }
          }
        }
        // Transposing V^T reads and P^T reads are issued through inline asm (the
        // compiler would order the intrinsic after every in-flight global->LDS
        // copy); completion is tracked here with lgkmcnt. Issue order: the 2 NVB
        // V^T halves, then P^T of row blocks 0 .. PPF - 1; row block rb + PPF is
        // issued after row block rb is consumed.
        lgkm_wait_n<0>();
        constexpr int PPF = 2;
        u32x4_t vf[NVB];
        u32x4_t pf[PPF];
        static_for<0, NVB>([&](auto VB) {
          constexpr int vb = decltype(VB)::value;
          const uint32_t a = vaddr(vb) + boff;
          const u32x2_t r0 = ds_read_tr16_b64_asm<0>(a);
          const u32x2_t r1 = ds_read_tr16_b64_asm<ROW16>(a);
          vf[vb] = u32x4_t{r0[0], r0[1], r1[0], r1[1]};
        });
        static_for<0, PPF>([&](auto RB) {
          constexpr int rb = decltype(RB)::value;
          pf[rb] = ds_read_b128_asm<rb * 1024>(paddr);
        });
        static_for<0, NRB>([&](auto RB) {
          constexpr int rb = decltype(RB)::value;
          constexpr int newer = (NRB - 1 - rb) < (PPF - 1) ? (NRB - 1 - rb) : (PPF - 1);
          lgkm_wait_n<newer>();
          __builtin_amdgcn_sched_barrier(0);
          if (rb < nrb) {
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) o[vb][rb] = DT::mfma16(vf[vb], pf[rb % PPF], o[vb][rb]);
          }
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (rb + PPF < NRB) pf[rb % PPF] = ds_read_b128_asm<(rb + PPF) * 1024>(paddr);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
    }

    // Denominators: the four lanes of a row hold partial sums of its keys.
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (q4 == 0) l_lds[rq] = l_tot;
    if (!whole && q4 == 0 && row_ok) {
      const int64_t slot = (int64_t)t.part_base + ((int)blockIdx.x - t.w_first);
      float* ml = p.part_ml + (slot * RW + rq) * 2;
      ml[0] = m_run;
      ml[1] = l_tot;
    }
    __syncthreads();   // denominators visible; LDS buffers free for the next piece

    // Lane holds O^T[channel VC w + 16 vb + 4 q4 + e][row 16 rb + l16].
    const int lane_e = opaque_lane();
    const int l16e = lane_e & 15, q4e = lane_e >> 4;
    if (whole) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const int r = 16 * rb + l16e;
        if (r < t.nrows) {
          const float lr = l_lds[r];
          const float inv = lr > 0.0f ? 1.0f / lr : 0.0f;
          const int R = t.row0 + r;
          const int tr = R / p.H;
          uint16_t* orow = p.out + ((int64_t)(cum_b + tr) * p.H + (R - tr * p.H)) * p.vhs;
          if (p.vhs == VHSP) {
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) {
              const int c = VC * w + 16 * vb + 4 * q4e;
              const uint32_t e0 = DT::from_f32(o[vb][rb][0] * inv), e1 = DT::from_f32(o[vb][rb][1] * inv);
              const uint32_t e2 = DT::from_f32(o[vb][rb][2] * inv), e3 = DT::from_f32(o[vb][rb][3] * inv);
              *(u32x2_t*)(orow + c) = u32x2_t{e0 | (e1 << 16), e2 | (e3 << 16)};
            }
          } else {
            for (int vb = 0; vb < NVB; ++vb)
              for (int e = 0; e < 4; ++e) {
                const int c = VC * w + 16 * vb + 4 * q4e + e;
                if (c < p.vhs) orow[c] = (uint16_t)DT::from_f32(o[vb][rb][e] * inv);
              }
          }
        }
      }
    } else {
      const int64_t slot = (int64_t)t.part_base + ((int)blockIdx.x - t.w_first);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const int r = 16 * rb + l16e;
        if (r < t.nrows) {
          float* acc = p.part_acc + slot * p.part_slot + (int64_t)r * p.part_row + VC * w + 4 * q4e;
#pragma unroll
          for (int vb = 0; vb < NVB; ++vb) *(f32x4_t*)(acc + 16 * vb) = o[vb][rb];
        }
      }
    }
    u = ub;
    ++i;
  }
#endif  // __HIP_DEVICE_COMPILE__
}

}  // namespace pa

#define PA_DEFINE_ATTN_WIDE_INSTANCE(DT, DTN, HSP, VHSP, KT, NB)                                            \
  namespace pa {                                                                                            \
  hipError_t PA_ATTN_FN(DTN, HSP, VHSP, 8, KT, occ)(int* n) {                                               \
    void (*fn)(AttnParams) = attn_wide_kernel<DT, HSP, VHSP, KT, NB>;                                       \
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, reinterpret_cast<const void*>(fn), 512, 0);      \
  }                                                                                                         \
  hipError_t PA_ATTN_FN(DTN, HSP, VHSP, 8, KT, launch)(const AttnParams& p, int grid, bool combine,          \
                                                       int cgrid, hipStream_t s) {                          \
    attn_wide_kernel<DT, HSP, VHSP, KT, NB><<<grid, 512, 0, s>>>(p);                                        \
    hipError_t e = hipGetLastError();                                                                       \
    if (e != hipSuccess || !combine) return e;                                                              \
    combine_kernel<DT, VHSP, 128><<<dim3(cgrid, 128 / kCombineRows), 256, 0, s>>>(p);                       \
    return hipGetLastError();                                                                               \
  }                                                                                                         \
  }
