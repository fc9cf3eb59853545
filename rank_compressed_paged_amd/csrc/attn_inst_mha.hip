// Attention instances for multi-head layers of any head count: up to 16 or
// 32 query heads (H and H_kv = H are kernel arguments) at r_k in {16, 32, 64}.
#include "attn_kernel.h"

namespace starkv {

bool attn_entry_mha(const AttnKey& key, AttnEntry& e) {
  STARKV_ATTN_RV(STARKV_ATTN_ENTRY, 32, 64, 8, 0, 0, 0)
  STARKV_ATTN_RV(STARKV_ATTN_ENTRY, 32, 32, 8, 0, 0, 0)
  STARKV_ATTN_RV(STARKV_ATTN_ENTRY, 32, 16, 8, 0, 0, 0)
  STARKV_ATTN_RV(STARKV_ATTN_ENTRY, 16, 64, 8, 0, 0, 0)
  STARKV_ATTN_RV(STARKV_ATTN_ENTRY, 16, 32, 8, 0, 0, 0)
  STARKV_ATTN_RV(STARKV_ATTN_ENTRY, 16, 16, 8, 0, 0, 0)
  return false;
}

}  // namespace starkv
