// Read phase, paired-workgroup variant for wide latent rows (576/512): each
// query tile of 128 rows is processed by two workgroups, one per half of the
// rows, that walk the same KV range. A workgroup has four waves of 16 query
// rows and uses v_mfma_f32_16x16x32; per wave the state is the 16 RoPE'd
// query rows (B fragments, HSP/32 x 4 VGPRs) and the transposed output
// accumulators (VHSP/16 x 4), about 200 registers, so nothing spills.
//
// The two workgroups of a pair have ids i and i + 8 (mod 16), which the
// dispatcher places on the same XCD: the second read of each KV tile is served
// by that XCD's L2, so HBM traffic stays one pass over the cache while the LDS
// and register state per CU halves.
//
// Semantics are those of attn_kernel (pa_attn.cuh): docs.rs page
// "onnx-runtime-ep-cuda src/kernels/paged_attention.rs", "LATENT semantics",
// read phase (device function attn_impl).
#pragma once

#include "pa_attn.cuh"

namespace pa {

template <typename DT, int HSP, int VHSP, int KT>
struct WaveState16 {
  static constexpr int NKK = HSP / 32;
  static constexpr int NMT = VHSP / 16;
  u32x4_t qf[NKK];
  f32x4_t o[NMT];
  float m_run, l_run;
};

// S^T = K Q^T on 16x16x32 (16 keys x 16 rows per accumulator, 32 channels per
// step), softmax update, O^T += V^T P^T (16 channels x 16 rows, 32 keys per step).
template <typename DT, int HSP, int VHSP, int KT>
__device__ __forceinline__ void tile_compute16(WaveState16<DT, HSP, VHSP, KT>& st, const uint8_t* L, int key0,
                                               int pos, int lo_row, bool softcap_on, const AttnParams& p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int CPR = HSP / 8;
  constexpr int NKK = HSP / 32;     // channel steps
  constexpr int NSUB = KT / 16;     // 16-key accumulators
  constexpr int NKS = KT / 32;      // PV key steps
  constexpr int NMT = VHSP / 16;
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;

  // A fragment: key l16 (+16 sub), chunk 4 kk + q4. Chunks 8 apart share the
  // swizzle: two base addresses (kk parity) and immediate offsets.
  const int swk = lds_swizzle(l16);
  const uint8_t* kb[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) kb[r] = L + l16 * CPR * 16 + (((4 * r + q4) ^ swk) << 4);
  // Step n: channel step kk = n / NSUB, accumulator sub = n % NSUB; even and
  // odd channel steps go to separate accumulators (summed afterwards), so at
  // least four independent MFMA chains interleave.
  constexpr int QPF = 8;
  constexpr int QSTEPS = NSUB * NKK;
  f32x4_t s[NSUB], s2[NSUB];
#pragma unroll
  for (int sub = 0; sub < NSUB; ++sub) { s[sub] = f32x4_t{0.f, 0.f, 0.f, 0.f}; s2[sub] = s[sub]; }
  auto k_frag = [&](int n) -> u32x4_t {
    const int kk = n / NSUB, sub = n % NSUB;
    return *(const u32x4_t*)(kb[kk & 1] + sub * 16 * CPR * 16 + (kk >> 1) * 128);
  };
  u32x4_t ka[QPF];
#pragma unroll
  for (int n = 0; n < QPF; ++n) ka[n] = k_frag(n);
#pragma unroll
  for (int n = 0; n < QSTEPS; ++n) {
    const u32x4_t cur = ka[n % QPF];
    if (n + QPF < QSTEPS) ka[n % QPF] = k_frag(n + QPF);
    const int kk = n / NSUB, sub = n % NSUB;
    if (kk & 1) s2[sub] = DT::mfma16(cur, st.qf[kk], s2[sub]);
    else s[sub] = DT::mfma16(cur, st.qf[kk], s[sub]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int sub = 0; sub < NSUB; ++sub) s[sub] += s2[sub];

  // Lane holds keys 16 sub + 4 q4 + i of its row l16.
  if (softcap_on) {
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub)
#pragma unroll
      for (int i = 0; i < 4; ++i) s[sub][i] = softcap_log2(s[sub][i], p.scale, p.softcap, p.softcap_inv);
  } else {
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) s[sub] *= p.scale_log2;
  }
  float tmax = -INFINITY;
#pragma unroll
  for (int sub = 0; sub < NSUB; ++sub) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = key0 + sub * 16 + q4 * 4 + i;
      const float v = (j <= pos && j >= lo_row) ? s[sub][i] : -INFINITY;
      s[sub][i] = v;
      tmax = fmaxf(tmax, v);
    }
  }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  const bool bump = tmax > st.m_run + 8.0f;
  const float m_new = bump ? tmax : st.m_run;
  const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
  const float corr = fast_exp2(st.m_run - m_use);
  const bool rescale = bump && (st.m_run != -INFINITY);
  st.m_run = m_new;
  // P^T for key step ks: k-index 8 q4 + e <-> key 32 ks + 4 q4 + (e & 3) + 16 (e >> 2),
  // i.e. accumulator 2 ks + (e >> 2), element e & 3.
  u32x4_t pf[NKS];
  float psum = 0.0f;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pv[e] = fast_exp2(s[2 * ks + (e >> 2)][e & 3] - m_use);
      psum += pv[e];
    }
    pf[ks] = pack8<DT>(pv);
  }
  st.l_run = st.l_run * corr + psum;
  if (__any(rescale)) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) st.o[mt] *= corr;
  }
  // V^T fragment (16 channels x 32 keys): transposing reads; lane (q4, jj, cq)
  // supplies key 32 ks + 4 q4 + jj + 16 r and channels 16 mt + 4 cq .. + 3.
  const int jj = (lane & 15) >> 2;
  const int cq = lane & 3;
  const int kr = 4 * q4 + jj;              // key within a 16-key half, < 16
  const int swv = lds_swizzle(kr);         // same for kr + 16 (period 16)
  // The transposing reads are issued through inline asm: the compiler treats
  // the intrinsic as aliasing every in-flight global->LDS copy and would wait
  // for the next tile's copy before each of them. Their completion is tracked
  // here instead: step n's two reads are followed by at most 2 * (VPF - 1)
  // newer LDS operations when step n is consumed (no scalar loads are in
  // flight in this loop), so lgkmcnt(2 * (VPF - 1)) orders them.
  uint32_t vb[4];
#pragma unroll
  for (int m4 = 0; m4 < 4; ++m4)
    vb[m4] = lds_addr(L + kr * CPR * 16 + (((2 * m4 + (cq >> 1)) ^ swv) << 4) + (cq & 1) * 8);
  constexpr int VPF = 8;
  constexpr int VSTEPS = NKS * NMT;
  static_assert(2 * (VPF - 1) <= 15, "lgkmcnt range");
  constexpr int ROW16 = 16 * CPR * 16;
  static_assert(ROW16 + (NKS - 1) * 32 * CPR * 16 + (NMT / 4 - 1) * 128 < 65536, "ds offset range");
  lgkm_wait_n<0>();   // no scalar load may be in flight while lgkmcnt counts LDS reads
  u32x4_t va[VPF];
  auto v_issue = [&](auto N) {
    constexpr int n = decltype(N)::value;
    constexpr int ks = n / NMT, mt = n % NMT;
    constexpr int off = ks * 32 * CPR * 16 + (mt >> 2) * 128;
    const u32x2_t r0 = ds_read_tr16_b64_asm<off>(vb[mt & 3]);
    const u32x2_t r1 = ds_read_tr16_b64_asm<off + ROW16>(vb[mt & 3]);
    va[n % VPF] = u32x4_t{r0[0], r0[1], r1[0], r1[1]};
  };
  static_for<0, VPF>(v_issue);
  static_for<0, VSTEPS>([&](auto N) {
    constexpr int n = decltype(N)::value;
    constexpr int left = VSTEPS - 1 - n;
    lgkm_wait_n<2 * (left < VPF - 1 ? left : VPF - 1)>();
    __builtin_amdgcn_sched_barrier(0);
    st.o[n % NMT] = DT::mfma16(va[n % VPF], pf[n / NMT], st.o[n % NMT]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (n + VPF < VSTEPS) v_issue(std::integral_constant<int, n + VPF>{});
    __builtin_amdgcn_sched_barrier(0);
  });
#endif  // __HIP_DEVICE_COMPILE__
}

// Workgroup i handles rows [64 h, 64 h + 64) of every query tile in unit range
// k, with h = (i >> 3) & 1 and k = (i >> 4) * 8 + (i & 7): the pair (i, i + 8)
// lands on one XCD. The schedule's ranges are indexed by k. NBUF LDS tile
// buffers keep up to NBUF - 1 tiles of copies in flight per workgroup.
template <typename DT, int HSP, int VHSP, int KT, int NBUF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1))) void attn16_kernel(AttnParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NW = 4;
  constexpr int CPR = HSP / 8;
  constexpr int TILE_CHUNKS = KT * CPR;
  constexpr int NT = NW * 64;
  constexpr int LOADS = TILE_CHUNKS / NT;
  constexpr int NKK = HSP / 32;
  constexpr int NMT = VHSP / 16;
  constexpr int RW = 128;              // rows of a query tile (both halves)
  constexpr int HALF = 64;
  static_assert(HSP % 64 == 0 && VHSP % 16 == 0 && VHSP <= HSP && KT % 32 == 0 && TILE_CHUNKS % NT == 0, "shape");
  constexpr int QSTRIDE = HSP + 8;
  constexpr int BUF_BYTES = TILE_CHUNKS * 16;
  constexpr int QSTAGE_BYTES = HALF * QSTRIDE * 2;
  constexpr int LDS_BYTES = (NBUF * BUF_BYTES > QSTAGE_BYTES) ? NBUF * BUF_BYTES : QSTAGE_BYTES;
  static_assert(NBUF >= 2 && (NBUF - 2) * (KT * CPR / (4 * 64)) <= 63, "vmcnt range");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[LDS_BYTES];

  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int q4 = lane >> 4;
  const int half = (blockIdx.x >> 3) & 1;
  const int range = (int)((blockIdx.x >> 4) << 3) + (int)(blockIdx.x & 7);

  int u = ld_uniform(p.wg_range + range);
  const int u_end = ld_uniform(p.wg_range + range + 1);
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
  // Wave w copies LDS slots [w * LOADS * 64, (w + 1) * LOADS * 64): keys
  // [w * KW, (w + 1) * KW) of the tile, KW = KT / NW <= 16 keys, which always lie
  // in one cache block (block_size >= 16, a power of two). Byte offset of each lane's chunk
  // relative to the first of those keys' rows (tile-independent).
  constexpr int KW = KT / NW;
  static_assert(KW * CPR == LOADS * 64 && KW <= 16, "one block slice per wave (block_size >= 16)");
  int load_off[LOADS];
#pragma unroll
  for (int it = 0; it < LOADS; ++it) {
    const int sl = it * 64 + lane;            // slot within the wave's slice
    const int k = sl / CPR;                   // key within the slice
    const int lc = (sl - k * CPR) ^ lds_swizzle(w * KW + k);
    load_off[it] = (k * p.hs + lc * 8) * 2;
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

    const int rloc = half * HALF + w * 16 + l16;     // row within the query tile
    const bool row_ok = rloc < t.nrows;
    const int R = t.row0 + rloc;
    const int tq = R / p.H;
    const int h = R - tq * p.H;
    const int pos = row_ok ? past_b + tq : -1;
    const int lo_row = p.window >= 0 ? max(0, pos - p.window) : 0;
    const bool wave_active = half * HALF + w * 16 < t.nrows;
    const int64_t qrow = (int64_t)(cum_b + tq) * p.H + h;

    WaveState16<DT, HSP, VHSP, KT> st;
    {
      // Stage this wave's 16 query rows in LDS, RoPE them there, read fragments
      // (row l16, channels 32 kk + 8 q4 .. + 8).
      uint16_t* qs = (uint16_t*)lds_raw + w * 16 * QSTRIDE;
      constexpr int QCH = HSP / 8;
      for (int idx = lane; idx < 16 * QCH; idx += 64) {
        const int r = idx / QCH;
        const int c0 = (idx - r * QCH) * 8;
        const int rl = half * HALF + w * 16 + r;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (rl < t.nrows && c0 < p.hs) {
          const int Rr = t.row0 + rl;
          const int tr = Rr / p.H;
          const int64_t gq = (int64_t)(cum_b + tr) * p.H + (Rr - tr * p.H);
          v = *(const u32x4_t*)(p.query + gq * p.hs + c0);
        }
        *(u32x4_t*)(qs + r * QSTRIDE + c0) = v;
      }
      __syncthreads();
      if (p.do_rotary) {
        const int hr = p.rd >> 1;
        for (int idx = lane; idx < 16 * hr; idx += 64) {
          const int r = idx / hr;
          const int k = idx - r * hr;
          const int rl = half * HALF + w * 16 + r;
          if (rl >= t.nrows) continue;
          const int posr = past_b + (t.row0 + rl) / p.H;
          const int d1 = p.interleaved ? p.ro + 2 * k : p.ro + k;
          const int d2 = p.interleaved ? d1 + 1 : d1 + hr;
          const float c = DT::to_f32(p.cos_t[(int64_t)posr * hr + k]);
          const float sn = DT::to_f32(p.sin_t[(int64_t)posr * hr + k]);
          const float x1 = DT::to_f32(qs[r * QSTRIDE + d1]);
          const float x2 = DT::to_f32(qs[r * QSTRIDE + d2]);
          qs[r * QSTRIDE + d1] = (uint16_t)DT::from_f32(x1 * c - x2 * sn);
          qs[r * QSTRIDE + d2] = (uint16_t)DT::from_f32(x2 * c + x1 * sn);
        }
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        st.qf[kk] = *(const u32x4_t*)(qs + l16 * QSTRIDE + 32 * kk + 8 * q4);
      __syncthreads();
    }
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) st.o[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    st.m_run = -INFINITY;
    st.l_run = 0.0f;

    // Every call issues exactly LOADS copy instructions per wave (the pipeline
    // below counts them with vmcnt); slots of keys outside [kv_lo, kv_hi) or of
    // channels >= hs copy 16 zero bytes from the workspace's zero page.
    // Block-table entry of this wave's slice of `tile` (scalar load).
    auto slice_block = [&](int tile) -> int {
      return ld_uniform(p.bt + (int64_t)b * p.MB + min((tile * KT + w * KW) >> p.bs_log2, p.MB - 1));
    };
    auto issue = [&](int tile, int bufi, int blk) {
      const int key0 = tile * KT;
      const int kw0 = key0 + w * KW;                       // first key of this wave's slice
      uint8_t* dst0 = lds_raw + bufi * BUF_BYTES + w * LOADS * 64 * 16;
      const uint8_t* base = (const uint8_t*)(p.cache + (((int64_t)blk << p.bs_log2) +
                                                        (kw0 & ((1 << p.bs_log2) - 1))) * p.hs);
      if (kw0 >= t.kv_lo && kw0 + KW <= t.kv_hi && p.hs == HSP) {
#pragma unroll
        for (int it = 0; it < LOADS; ++it)
          __builtin_amdgcn_global_load_lds(base + load_off[it], dst0 + it * 64 * 16, 16, 0, 0);
      } else {
#pragma unroll
        for (int it = 0; it < LOADS; ++it) {
          const int sl = it * 64 + lane;
          const int k = sl / CPR;
          const int lc = (sl - k * CPR) ^ lds_swizzle(w * KW + k);
          const int j = kw0 + k;
          const bool ok = j >= t.kv_lo && j < t.kv_hi && lc * 8 < p.hs;
          const uint8_t* src = ok ? base + load_off[it] : (const uint8_t*)p.zero16;
          __builtin_amdgcn_global_load_lds(src, dst0 + it * 64 * 16, 16, 0, 0);
        }
      }
    };

    // Copies of tiles tt + 1 .. tt + NBUF - 2 stay in flight while tile tt is
    // computed; loads complete in order, so vmcnt(ahead * LOADS) means tile tt
    // has landed. Buffer (tt - tile_a) % NBUF is refilled with tile
    // tt + NBUF - 1 only after the barrier that ends every wave's work on tile tt - 1.
    // The block-table entry of the tile issued in an iteration is loaded one
    // iteration earlier, so the scalar load's latency stays off the copy path;
    // the lgkmcnt(0) before the transposing reads of tile_compute16 retires it.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // drain the previous piece's stores
#pragma unroll
    for (int k = 0; k < NBUF - 1; ++k)
      if (tile_a + k < tile_b) issue(tile_a + k, k, slice_block(tile_a + k));
    int blk_next = slice_block(tile_a + NBUF - 1);
    for (int tt = tile_a; tt < tile_b; ++tt) {
      const int bufi = (tt - tile_a) % NBUF;
      const int ahead = min(NBUF - 2, tile_b - 1 - tt);
      vm_wait_tiles<LOADS, NBUF - 2>(ahead);
      __syncthreads();
      const int blk_cur = blk_next;
      blk_next = slice_block(tt + NBUF);
      if (tt + NBUF - 1 < tile_b) issue(tt + NBUF - 1, (tt + NBUF - 1 - tile_a) % NBUF, blk_cur);
      if (wave_active)
        tile_compute16<DT, HSP, VHSP, KT>(st, lds_raw + bufi * BUF_BYTES, tt * KT, pos, lo_row, softcap_on, p);
    }
    __syncthreads();

    float l_tot = st.l_run + __shfl_xor(st.l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (whole) {
      if (row_ok) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        uint16_t* orow = p.out + qrow * p.vhs;
        if (p.vhs == VHSP) {
          uint16_t* ob = orow + q4 * 4;
#pragma unroll
          for (int mt = 0; mt < NMT; ++mt) {
            const uint32_t e0 = DT::from_f32(st.o[mt][0] * inv), e1 = DT::from_f32(st.o[mt][1] * inv);
            const uint32_t e2 = DT::from_f32(st.o[mt][2] * inv), e3 = DT::from_f32(st.o[mt][3] * inv);
            *(u32x2_t*)(ob + mt * 16) = u32x2_t{e0 | (e1 << 16), e2 | (e3 << 16)};
          }
        } else {
          for (int mt = 0; mt < NMT; ++mt)
            for (int e = 0; e < 4; ++e) {
              const int c = mt * 16 + q4 * 4 + e;
              if (c < p.vhs) orow[c] = (uint16_t)DT::from_f32(st.o[mt][e] * inv);
            }
        }
      }
    } else {
      const int64_t slot = (int64_t)t.part_base + (range - t.w_first);
      if (q4 == 0) {
        float* ml = p.part_ml + (slot * RW + rloc) * 2;
        ml[0] = st.m_run;
        ml[1] = l_tot;
      }
      float* acc = p.part_acc + (slot * RW + rloc) * VHSP + q4 * 4;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) *(f32x4_t*)(acc + mt * 16) = st.o[mt];
    }
    u = ub;
    ++i;
  }
#endif  // __HIP_DEVICE_COMPILE__
}

}  // namespace pa

#define PA_DEFINE_ATTN16_INSTANCE(DT, DTN, HSP, VHSP, KT, NBUF)                                                  \
  namespace pa {                                                                                            \
  hipError_t PA_ATTN_FN(DTN, HSP, VHSP, 16, KT, occ)(int* n) {                                              \
    void (*fn)(AttnParams) = attn16_kernel<DT, HSP, VHSP, KT, NBUF>;                                              \
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, reinterpret_cast<const void*>(fn), 256, 0);      \
  }                                                                                                         \
  hipError_t PA_ATTN_FN(DTN, HSP, VHSP, 16, KT, launch)(const AttnParams& p, int grid, bool combine,         \
                                                        int cgrid, hipStream_t s) {                           \
    attn16_kernel<DT, HSP, VHSP, KT, NBUF><<<grid, 256, 0, s>>>(p);                                               \
    hipError_t e = hipGetLastError();                                                                       \
    if (e != hipSuccess || !combine) return e;                                                              \
    combine_kernel<DT, VHSP, 128><<<dim3(cgrid, 128 / kCombineRows), 256, 0, s>>>(p);                        \
    return hipGetLastError();                                                                               \
  }                                                                                                         \
  }
