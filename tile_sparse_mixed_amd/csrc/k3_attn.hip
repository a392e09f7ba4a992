// Dispatch of the fused three-tier pass (K3) to the translation unit of the
// plan's key-block size; the kernel itself is in k3_attn.hpp.
#include "tattn_internal.hpp"

namespace tattn {

hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  switch (a.d.Bk) {
    case 64: return launch_attn_bk64(a, s);
    case 16: return launch_attn_bk16(a, s);
    case 8: return launch_attn_bk8(a, s);
    case 4: return launch_attn_bk4(a, s);
    case 2: return launch_attn_bk2(a, s);
    case 1: return launch_attn_bk1(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tattn
