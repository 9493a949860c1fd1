// Explicit instances of the decode launches (kernels in decode_impl.h).  The build compiles this
// file once per (head_dim, group, cold-tile format) with HKV_D, HKV_G and HKV_BITS defined, so the
// instances compile in parallel; without them it instantiates every one.
#include "decode_impl.h"

namespace hkv {

#if defined(HKV_D) && defined(HKV_G) && defined(HKV_BITS)
template hipError_t launch_decode_dgb<HKV_D, HKV_G, HKV_BITS>(const DecodeParams&, const LaunchCtx&, const uint16_t*);
#else
#define HKV_INST(D, G, BITS) \
  template hipError_t launch_decode_dgb<D, G, BITS>(const DecodeParams&, const LaunchCtx&, const uint16_t*);
#define HKV_INST_D(D, BITS) HKV_INST(D, 1, BITS) HKV_INST(D, 2, BITS) HKV_INST(D, 4, BITS) HKV_INST(D, 8, BITS)
HKV_INST_D(128, 8) HKV_INST_D(64, 8) HKV_INST_D(128, 4) HKV_INST_D(64, 4) HKV_INST_D(128, 0) HKV_INST_D(64, 0)
#endif

}  // namespace hkv
