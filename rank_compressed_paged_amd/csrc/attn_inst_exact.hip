// Attention instances built for exact head counts (the counts are constants
// in the code): 32-head layers at every built rank, grouped 32/8 and 32/4
// layers, and the two small parity shapes.
#include "attn_kernel.h"

namespace starkv {

bool attn_entry_exact(const AttnKey& key, AttnEntry& e) {
  STARKV_ATTN_RV(STARKV_ATTN_ENTRY, 32, 64, 8, 0, 32, 32)
  STARKV_ATTN_RV(STARKV_ATTN_ENTRY, 32, 32, 8, 0, 32, 32)
  STARKV_ATTN_RV(STARKV_ATTN_ENTRY, 32, 16, 8, 0, 32, 32)
  STARKV_ATTN_RV(STARKV_ATTN_ENTRY, 32, 64, 8, 2, 32, 8)
  STARKV_ATTN_RV(STARKV_ATTN_ENTRY, 32, 32, 8, 1, 32, 8)
  STARKV_ATTN_RV(STARKV_ATTN_ENTRY, 32, 64, 8, 1, 32, 4)
  STARKV_ATTN_ENTRY(4, 16, 64, 2, 0, 4, 4)
  STARKV_ATTN_ENTRY(8, 32, 64, 2, 1, 8, 2)
  return false;
}

}  // namespace starkv
