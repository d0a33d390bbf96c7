// libbiwkv translation unit: Bi-WKV tile-kernel launches for fp32 k and v.
#include "row_launch.h"

namespace biwkv_host {

int forward_f32(const BiwkvParams& bp, int64_t B, int kind, int dev, void* stream, const FixedScratch* fixed) {
  return forward_kind<BIWKV_F32, false>(bp, B, kind, dev, stream, fixed);
}

}  // namespace biwkv_host
