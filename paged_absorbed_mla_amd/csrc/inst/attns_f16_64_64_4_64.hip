// Attention instance, separate (grouped-query) layout: f16 storage, key/value head sizes
// padded to 64/64, 4 waves, 64-key tiles, query channels [0, 64) held in registers.
#include "../pa_attn.cuh"

PA_DEFINE_ATTN_INSTANCE(sep, F16, f16, 64, 64, 4, 64, 64)
