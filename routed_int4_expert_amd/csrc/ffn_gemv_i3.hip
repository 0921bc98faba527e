// ffn_gemv_i3.hip -- the int3-g64 instantiation of the grouped dequantising GEMVs
// (ffn_gemv.h), in a translation unit of its own so the formats compile in parallel.
#include "ffn_gemv.h"

namespace moe {

template hipError_t gemv_dispatch<kFmtI3>(bool, const FfnArgs &, int, int, int, hipStream_t);

}  // namespace moe
