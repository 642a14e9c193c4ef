// Attention instance: bf16 storage, head sizes padded to 576/512, paired workgroups of
// four 16-row waves, 64-key tiles, 2 LDS tile buffers.
#include "../pa_attn16.cuh"

PA_DEFINE_ATTN16_INSTANCE(BF16, bf16, 576, 512, 64, 2)
