// Attention instance: bf16 storage, head sizes padded to 192/128, 4 waves, 64-key tiles.
#include "../pa_attn.cuh"

PA_DEFINE_ATTN_INSTANCE(BF16, bf16, 192, 128, 4, 64)
