// Write phase: partial RoPE of each new latent key row, scattered in place into
// the paged block cache at slot_mapping[t] (-1 skips).
//
// Semantics: docs.rs page "onnx-runtime-ep-cuda src/kernels/paged_attention.rs",
// "LATENT semantics" (write phase) and device function write_impl. The page's
// kernel runs one thread per element with a linear sequence scan per element;
// here one wavefront owns one token row: the (batch, position) lookup and the
// slot read happen once per row, and the row moves as coalesced 16-byte
// chunks (8 channels per lane).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kWriteWaves = 4;

template <typename DT>
__global__ __launch_bounds__(kWriteWaves * 64) void write_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ cos_t, const uint16_t* __restrict__ sin_t,
    const int32_t* __restrict__ slot_mapping, const int32_t* __restrict__ cumseq,
    const int32_t* __restrict__ past, uint16_t* __restrict__ cache, int64_t T, int rw, int hw, int ro, int rd,
    int do_rotary, int interleaved, int B, int64_t num_slots, int64_t prow) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kWriteWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const int slot = slot_mapping[t];
  // -1 skips the row; so does a slot past the cache (a violated precondition).
  if (slot < 0 || slot >= num_slots) return;
  const int b = find_seq(cumseq, B, t);
  // Position clamped into the rotary table (only a violated precondition moves it).
  const int64_t pos = min(max((int64_t)past[b] + (t - (int64_t)cumseq[b]), (int64_t)0), prow - 1);
  // A slot row holds rw / hw heads of hw channels each (one latent row, or
  // the key or value heads of the separate layout); RoPE applies per head.
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

template <typename DT>
static hipError_t write_rows(const CallGeom& g, const void* src, void* cache, int hw, int rotary, const void* cos_t,
                             const void* sin_t, const int32_t* slot, const int32_t* cumseq, const int32_t* past,
                             hipStream_t stream) {
  const int64_t blocks = (g.T + kWriteWaves - 1) / kWriteWaves;
  write_kernel<DT><<<dim3((unsigned)blocks), dim3(kWriteWaves * 64), 0, stream>>>(
      (const uint16_t*)src, (const uint16_t*)cos_t, (const uint16_t*)sin_t, slot, cumseq, past, (uint16_t*)cache,
      g.T, g.kvh * hw, hw, g.ro, g.rd, rotary, g.interleaved, g.B, g.NB * g.bs, g.do_rotary ? g.P : 1);
  return hipGetLastError();
}

hipError_t launch_write(const CallGeom& g, const void* key, const void* value, const void* cos_t,
                        const void* sin_t, const int32_t* slot, const int32_t* cumseq, const int32_t* past,
                        void* cache, void* value_cache, hipStream_t stream) {
  if (g.T == 0) return hipSuccess;
  auto run = [&](auto tag) -> hipError_t {
    using DT = decltype(tag);
    hipError_t e = write_rows<DT>(g, key, cache, g.hs, g.do_rotary, cos_t, sin_t, slot, cumseq, past, stream);
    if (e != hipSuccess || !g.sep) return e;
    // Value rows: stored unrotated.
    return write_rows<DT>(g, value, value_cache, g.vhs, 0, cos_t, sin_t, slot, cumseq, past, stream);
  };
  return g.dtype == 16 ? run(BF16{}) : run(F16{});
}

}  // namespace pa
