// Attention instance: f16 storage, head sizes padded to 64/32, 1 waves, 32-key tiles,
// query channels [0, 64) held in registers.
#include "../pa_attn.cuh"

PA_DEFINE_ATTN_INSTANCE(lat, F16, f16, 64, 32, 1, 32, 64)
