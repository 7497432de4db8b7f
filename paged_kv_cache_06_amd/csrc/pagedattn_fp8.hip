// libpagedattn, decode attention over E4M3 (FP8) pools: the instances of
// decode_kernel for pools of 8-bit floats, in their own translation unit so
// that the two sets compile in parallel. The host side (argument checks,
// workspace, launch) is shared with the fp16 pools in pagedattn.hip.

#include "decode_kernel.h"

namespace pa_detail {

DecodeFn pick_decode_fp8(int bs, int D, int nrep) { return pick_decode_t<true>(bs, D, nrep); }

}  // namespace pa_detail
