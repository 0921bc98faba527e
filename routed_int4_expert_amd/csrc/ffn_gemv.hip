// ffn_gemv.hip -- the grouped dequantising GEMVs of ffn_gemv.h: the int4-gs64 kernels,
// the opt-in 8-bit activation pre-pass and the launch sequence of the expert FFNs for
// a few tokens (every expert format).
#include "ffn_gemv.h"

namespace moe {

template hipError_t gemv_dispatch<kFmtI4>(bool, const FfnArgs &, int, int, int, hipStream_t);

int rows_per_pass(int T, int K, int fmt) {
    (void)fmt;  // every format stages the same 16-bit chunks
    const size_t row_bytes = (size_t)(K / 32) * kChunkPitch * sizeof(float);
    int rm = T >= 3 ? 4 : (T == 2 ? 2 : 1);
    while (rm > 1 && (size_t)rm * row_bytes > 160 * 1024) rm >>= 1;
    return rm;
}

static hipError_t dispatch(bool GU, const FfnArgs &a, int N, int K, int rm, hipStream_t st) {
    if (a.fmt == kFmtF4) return gemv_dispatch<kFmtF4>(GU, a, N, K, rm, st);
    if (a.fmt == kFmtI3) return gemv_dispatch<kFmtI3>(GU, a, N, K, rm, st);
    return gemv_dispatch<kFmtI4>(GU, a, N, K, rm, st);
}

// The opt-in 8-bit activations on this path: rows of K values replaced, per block of 32
// (the staging chunk), by c * 2^-n with c = rint(x * 2^n) in [-127, 127] and n the 8-bit
// rule's shift (act_shift).  The kernels above then stage such a block exactly: its
// 16-bit shift is n + 8 (max|c| is in [64, 127]), so x16 = 256 c, hi = c and lo = 0, and the
// integer products equal those of the 8-bit codes.  One thread per block; dst may alias src.
__global__ __launch_bounds__(256) void quant_act8_kernel(const float *src, float *dst, int rows, int K) {
    const int nb = K / 32;
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= rows * nb) return;
    const float4 *p = reinterpret_cast<const float4 *>(src + (size_t)(b / nb) * K + 32 * (b % nb));
    float4 v[8];
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = p[i];
    uint32_t mb = 0;
#pragma unroll
    for (int i = 0; i < 8; i++)
        mb = max(mb, max(max(__float_as_uint(v[i].x) & 0x7FFFFFFFu, __float_as_uint(v[i].y) & 0x7FFFFFFFu),
                         max(__float_as_uint(v[i].z) & 0x7FFFFFFFu, __float_as_uint(v[i].w) & 0x7FFFFFFFu)));
    const bool finite = mb < 0x7F800000u;
    const int n = (finite && mb) ? act_shift(mb, act_rule(1)) : 0;
    auto q = [&](float x) __attribute__((always_inline)) {
        if (!finite) return __int_as_float(0x7FC00000);  // a non-finite block stays non-finite
        return ldexpf(fminf(fmaxf(rintf(ldexpf(x, n)), -127.0f), 127.0f), -n);
    };
    float4 *o = reinterpret_cast<float4 *>(dst + (size_t)(b / nb) * K + 32 * (b % nb));
#pragma unroll
    for (int i = 0; i < 8; i++) o[i] = make_float4(q(v[i].x), q(v[i].y), q(v[i].z), q(v[i].w));
}

static hipError_t launch_quant_act8(const float *src, float *dst, int rows, int K, hipStream_t st) {
    const int n = rows * (K / 32);
    if (n <= 0) return hipSuccess;
    ProfScope prof("quant_act8", st);
    quant_act8_kernel<<<(n + 255) / 256, 256, 0, st>>>(src, dst, rows, K);
    return hipGetLastError();
}

static hipError_t launch_ffn_gemv_16(const FfnArgs &a, hipStream_t st);
static hipError_t launch_ffn_gemv_16_gateup(const FfnArgs &a, hipStream_t st);
static hipError_t launch_ffn_gemv_16_down(const FfnArgs &a, hipStream_t st);

// The opt-in 8-bit path: x quantised into the workspace, the gate/up kernels, h
// quantised in place, the down kernels.
hipError_t launch_ffn_gemv(const FfnArgs &a, hipStream_t st) {
    if (!a.act8) return launch_ffn_gemv_16(a, st);
    FfnArgs q = a;
    hipError_t e = launch_quant_act8(a.x, a.xq, a.T, a.H, st);
    q.x = a.xq;
    if (e == hipSuccess) e = launch_ffn_gemv_16_gateup(q, st);
    if (e == hipSuccess && a.with_routed) e = launch_quant_act8(a.h_routed, a.h_routed, a.rows_max, a.F, st);
    if (e == hipSuccess && a.with_shared) e = launch_quant_act8(a.h_shared, a.h_shared, a.T, a.Fs, st);
    if (e == hipSuccess) e = launch_ffn_gemv_16_down(q, st);
    return e;
}

// Gate/up then down.  Routed and shared units share a launch when their
// reduction lengths give the same lane split; otherwise each has its own.
static hipError_t launch_ffn_gemv_16(const FfnArgs &a, hipStream_t st) {
    hipError_t e = launch_ffn_gemv_16_gateup(a, st);
    if (e != hipSuccess) return e;
    return launch_ffn_gemv_16_down(a, st);
}

static hipError_t launch_ffn_gemv_16_gateup(const FfnArgs &a, hipStream_t st) {
    const int nmax = a.with_shared ? (a.with_routed ? max(a.F, a.Fs) : a.Fs) : a.F;
    return dispatch(true, a, nmax, a.H, rows_per_pass(a.T, a.H, a.fmt), st);
}

static hipError_t launch_ffn_gemv_16_down(const FfnArgs &a, hipStream_t st) {
    hipError_t e;
    const bool same_down = !a.with_shared || !a.with_routed ||
                           lanes_per_row(a.F) == lanes_per_row(a.Fs);
    if (same_down) {
        // one launch; the LDS is sized for the longer of the two reductions
        const int K = a.with_routed ? a.F : a.Fs;
        const int kmax = a.with_shared && a.with_routed ? max(a.F, a.Fs) : K;
        return dispatch(false, a, a.H, kmax, rows_per_pass(a.T, kmax, a.fmt), st);
    }
    FfnArgs r = a;
    r.with_shared = 0;
    e = dispatch(false, r, a.H, a.F, rows_per_pass(a.T, a.F, a.fmt), st);
    if (e != hipSuccess) return e;
    FfnArgs s = a;
    s.with_routed = 0;
    return dispatch(false, s, a.H, a.Fs, rows_per_pass(a.T, a.Fs, a.fmt), st);
}

}  // namespace moe
