// The fused pass's instances with 64-key blocks (one translation unit per
// key-block size, so that the instances compile in parallel).
#include "k3_attn.hpp"

namespace tattn {
hipError_t launch_attn_bk64(const AttnArgs& a, hipStream_t s) { return launch_bk<64>(a, s); }
}  // namespace tattn
