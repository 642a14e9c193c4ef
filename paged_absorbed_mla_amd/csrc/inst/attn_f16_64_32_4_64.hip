// Attention instance: f16 storage, head sizes padded to 64/32, 4 waves, 64-key tiles,
// query channels [0, 64) held in registers.
#include "../pa_attn.cuh"

PA_DEFINE_ATTN_INSTANCE(lat, F16, f16, 64, 32, 4, 64, 64)
