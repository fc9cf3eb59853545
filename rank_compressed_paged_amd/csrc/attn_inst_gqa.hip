// Attention instances for grouped-query layers of any shape up to 32 query
// heads (H and H_kv are kernel arguments), with 1, 2 or 4 MFMA score units
// (key head, 32-latent k-step) per wave and block.
#include "attn_kernel.h"

namespace starkv {

bool attn_entry_gqa(const AttnKey& key, AttnEntry& e) {
  STARKV_ATTN_RV(STARKV_ATTN_ENTRY, 32, 64, 8, 1, 0, 0)
  STARKV_ATTN_RV(STARKV_ATTN_ENTRY, 32, 64, 8, 2, 0, 0)
  STARKV_ATTN_RV(STARKV_ATTN_ENTRY, 32, 64, 8, 4, 0, 0)
  STARKV_ATTN_RV(STARKV_ATTN_ENTRY, 32, 32, 8, 1, 0, 0)
  STARKV_ATTN_RV(STARKV_ATTN_ENTRY, 32, 32, 8, 2, 0, 0)
  return false;
}

}  // namespace starkv
