// libbiwkv translation unit: Bi-WKV tile-kernel launches for bf16 k and v loaded as 32-bit channel pairs.
#include "row_launch.h"

namespace biwkv_host {

int forward_bf16_pair(const BiwkvParams& bp, int64_t B, int kind, int dev, void* stream, const FixedScratch* fixed) {
  return forward_kind<BIWKV_BF16, true>(bp, B, kind, dev, stream, fixed);
}

}  // namespace biwkv_host
