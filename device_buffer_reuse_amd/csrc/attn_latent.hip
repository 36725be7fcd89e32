// Latent-layout attention (one shared latent KV head, many query heads).
#include "avsg_internal.h"

namespace avsg {

hipError_t launch_attn_latent(const AttnParams&, int, int, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace avsg
