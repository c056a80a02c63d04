// MFMA split-KV tree-verify kernel (bf16, head_dim 128) - under construction.
#include "launch.h"

namespace ta {

hipError_t launch_verify_mfma(const VerifyParams& p, hipStream_t stream) {
  (void)p;
  (void)stream;
  return hipErrorNotSupported;
}

}  // namespace ta
