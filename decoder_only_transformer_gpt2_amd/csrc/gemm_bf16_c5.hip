// bf16 GEMM, tile configuration 5 of the table in gemm_bf16_impl.h (own translation unit: the
// configurations compile in parallel).
#include "gemm_bf16_impl.h"

namespace gpt2k {
GPT2_GEMM_DEFINE_CFG(5)
}  // namespace gpt2k
