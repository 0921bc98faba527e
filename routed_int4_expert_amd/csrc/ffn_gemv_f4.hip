// ffn_gemv_f4.hip -- the MXFP4 instantiation of the grouped dequantising GEMVs
// (ffn_gemv.h), in a translation unit of its own so the formats compile in parallel.
#include "ffn_gemv.h"

namespace moe {

template hipError_t gemv_dispatch<kFmtF4>(bool, const FfnArgs &, int, int, int, hipStream_t);

}  // namespace moe
