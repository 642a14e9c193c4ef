// Write phase, one token row: partial RoPE of the new key row, scattered in
// place into the paged block cache at slot_mapping[t] (-1 skips).
//
// Semantics: docs.rs page "onnx-runtime-ep-cuda src/kernels/paged_attention.rs",
// "LATENT semantics" (write phase) and device function write_impl. The page's
// kernel runs one thread per element with a linear sequence scan per element;
// here one wavefront owns one token row: the (batch, position) lookup and the
// slot read happen once per row, and the row moves as coalesced 16-byte
// chunks (8 channels per lane). Used by the write launch and by the write
// blocks of the fused call's schedule launch.
#pragma once

#include "pa_device.h"

namespace pa {

// Row t of `key` ([T, rw]; a slot row holds rw / hw heads of hw channels each:
// one latent row, or the key or value heads of the separate layout; RoPE
// applies per head to channels [ro, ro + rd) when `do_rotary`) into cache row
// slot_mapping[t]. `lane`: the thread's lane in its wavefront.
template <typename DT>
__device__ __forceinline__ void write_row(const uint16_t* __restrict__ key, const uint16_t* __restrict__ cos_t,
                                          const uint16_t* __restrict__ sin_t, const int32_t* __restrict__ slot_mapping,
                                          const int32_t* __restrict__ cumseq, const int32_t* __restrict__ past,
                                          uint16_t* __restrict__ cache, int64_t t, int rw, int hw, int ro, int rd,
                                          int do_rotary, int interleaved, int B, int64_t num_slots, int64_t prow,
                                          int lane) {
  const int slot = slot_mapping[t];
  // -1 skips the row; so does a slot past the cache (a violated precondition).
  if (slot < 0 || slot >= num_slots) return;
  const int b = find_seq(cumseq, B, t);
  // Position clamped into the rotary table (only a violated precondition moves it).
  const int64_t pos = min(max((int64_t)past[b] + (t - (int64_t)cumseq[b]), (int64_t)0), prow - 1);
  const uint16_t* row = key + t * rw;
  uint16_t* dst = cache + (int64_t)slot * rw;
  const int nchunks = rw >> 3;
  for (int c = lane; c < nchunks; c += 64) {
    const int c0 = c << 3;
    u32x4_t v = *(const u32x4_t*)(row + c0);
    const int head = c0 / hw;
    const int hc = c0 - head * hw;
    if (do_rotary && hc >= ro && hc < ro + rd) {
      float x[8];
      unpack8<DT>(v, x);
      rope_chunk<DT>(x, row + head * hw, hc, ro, rd, interleaved, pos, cos_t, sin_t);
      v = pack8<DT>(x);
    }
    *(u32x4_t*)(dst + c0) = v;
  }
}

}  // namespace pa
