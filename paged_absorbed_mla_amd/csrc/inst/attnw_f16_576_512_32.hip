// Attention instance: f16 storage, head sizes padded to 576/512, eight waves per
// 128-row query tile, 32-key tiles, 4 LDS tile buffers.
#include "../pa_attn_wide.cuh"

PA_DEFINE_ATTN_WIDE_INSTANCE(F16, f16, 576, 512, 32, 4)
