// bf16 attention dispatch. The MFMA kernel replaces this forwarding shim.
#include <hip/hip_runtime.h>

#include "txl_internal.h"

namespace txl {

txl_status launch_rel_attn_mfma(const AttnParams &p, hipStream_t s) {
  return launch_rel_attn_valu(p, TXL_BF16, s);
}

}  // namespace txl
