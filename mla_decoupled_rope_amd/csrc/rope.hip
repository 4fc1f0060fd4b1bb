// K1: the decoupled RoPE channel and the paged latent-cache write.
//
// "AI decoupled RoPE MLA" (operatorworld.com), decoupled-RoPE section: only
// the d_r-wide q^R and k^R are rotated; "Latent Attention Meets RoPE", "Two
// small, telling details": the cache keeps the latent and one shared
// position key per token.  The key is stored already rotated to its own
// position, so decode needs no positions at all (R_m^T R_t depends only on
// t - m, "Detailed Illustration of the Problem", Step 3).
//
// A query n is one workgroup: every head of a query shares its position, so
// the d_r/2 angles are computed once (float64) into LDS and all heads'
// pairs are rotated from there with 16-byte loads and stores.  A cache row
// is one 64-lane wave: it copies c_t and writes R_t k^R_t into its page slot.
// Angles p * theta_j and sin / cos are float64 (positions reach 2^17, where a
// float32 angle would be off by ~1e-2 rad); the rotation is float64 too,
// rounded once to the output type.  The rotated query also takes the ratio
// of the position scale to the content scale (1 for one scale on the summed
// score), inside the same float64 product, so the two-scale score costs no
// extra rounding and no extra work in the attention kernels.
#include "rope_block.hpp"

namespace mla {

template <typename T, typename TQ>
__global__ void __launch_bounds__(256) rope_kernel(RopeParams p) {
  rope_block<T, TQ>(p, blockIdx.x);
}

hipError_t launch_rope(const RopeParams& p, hipStream_t s) {
  const int64_t blocks = rope_blocks(p);
  if (blocks == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (p.dtype == 0)
    hipLaunchKernelGGL((rope_kernel<float, float>), grid, dim3(256), 0, s, p);
  else if (p.work_dtype == 0)
    hipLaunchKernelGGL((rope_kernel<bf16_t, float>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((rope_kernel<bf16_t, bf16_t>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
