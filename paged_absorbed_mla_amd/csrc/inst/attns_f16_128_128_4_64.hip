// Attention instance, separate (grouped-query) layout: f16 storage, key/value head sizes
// padded to 128/128, 4 waves, 64-key tiles, query channels [0, 128) held in registers.
#include "../pa_attn.cuh"

PA_DEFINE_ATTN_INSTANCE(sep, F16, f16, 128, 128, 4, 64, 128)
