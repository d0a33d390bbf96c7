// libbiwkv translation unit: Bi-WKV tile-kernel launches for bf16 k and v loaded as 16-bit values (odd C or 2-byte alignment).
#include "row_launch.h"

namespace biwkv_host {

int forward_bf16(const BiwkvParams& bp, int64_t B, int kind, int dev, void* stream, const FixedScratch* fixed) {
  return forward_kind<BIWKV_BF16, false>(bp, B, kind, dev, stream, fixed);
}

}  // namespace biwkv_host
