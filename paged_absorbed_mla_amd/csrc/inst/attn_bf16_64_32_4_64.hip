// Attention instance: bf16 storage, head sizes padded to 64/32, 4 waves, 64-key tiles,
// query channels [0, 64) held in registers.
#include "../pa_attn.cuh"

PA_DEFINE_ATTN_INSTANCE(lat, BF16, bf16, 64, 32, 4, 64, 64)
