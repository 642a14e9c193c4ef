// Attention instance: f16 storage, head sizes padded to 576/512, four waves of 32 query
// rows with the query resident in registers, 32-key tiles, 4 LDS tile buffers.
#include "../pa_attn_mla.cuh"

PA_DEFINE_ATTN_MLA_INSTANCE(F16, f16, 576, 512)
