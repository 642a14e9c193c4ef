// Attention instance, separate (grouped-query) layout: f16 storage, key/value head sizes
// padded to 64/64, 1 wave, 32-key tiles, query channels [0, 64) held in registers.
#include "../pa_attn.cuh"

PA_DEFINE_ATTN_INSTANCE(sep, F16, f16, 64, 64, 1, 32, 64)
