// Write launch: one wavefront per token row (write_row in pa_write.cuh).
#include "pa_write.cuh"
#include "pa_internal.h"

namespace pa {

constexpr int kWriteWaves = 4;

template <typename DT>
__global__ __launch_bounds__(kWriteWaves * 64) void write_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ cos_t, const uint16_t* __restrict__ sin_t,
    const int32_t* __restrict__ slot_mapping, const int32_t* __restrict__ cumseq,
    const int32_t* __restrict__ past, uint16_t* __restrict__ cache, int64_t T, int rw, int hw, int ro, int rd,
    int do_rotary, int interleaved, int B, int64_t num_slots, int64_t prow) {
  const int64_t t = (int64_t)blockIdx.x * kWriteWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  write_row<DT>(key, cos_t, sin_t, slot_mapping, cumseq, past, cache, t, rw, hw, ro, rd, do_rotary, interleaved, B,
                num_slots, prow, threadIdx.x & 63);
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
