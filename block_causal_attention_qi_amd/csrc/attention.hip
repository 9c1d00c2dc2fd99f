// Translation unit of the attention kernel.  It is compiled with
// -amdgpu-mfma-vgpr-form: with two waves per SIMD and 256 registers each, the
// score and output accumulators must share the VGPR file with the softmax
// state; in the default (AGPR) form the compiler spills.
#include "attention.hpp"

void launch_block_causal_attn(const AttnBatch &ab, hipStream_t s) {
  const AttnArgs &a = ab.br[0];
  hipLaunchKernelGGL(block_causal_attn_kernel, dim3(a.n_img_qt + a.n_txt_qt, a.heads * ab.nbranch),
                     dim3(attn::THREADS), 0, s, ab);
}
