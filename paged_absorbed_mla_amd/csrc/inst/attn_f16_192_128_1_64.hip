// Attention instance: f16 storage, head sizes padded to 192/128, 1 waves, 64-key tiles,
// query channels [0, 192) held in registers.
#include "../pa_attn.cuh"

PA_DEFINE_ATTN_INSTANCE(lat, F16, f16, 192, 128, 1, 64, 192)
