// Value compression for gfx950 (discosf.com TurboQuant article, section
// "TurboQuant in one sentence", step 4: grouped 2/4-bit quantisation with bit
// packing).  One thread owns one (token, group): it loads the group with
// 16-byte loads, takes min/max, rounds scale and zero straight from fp64 to
// fp16, and writes whole packed words; adjacent threads write adjacent words.
#include "tq_internal.h"
#include "tq_device.h"

namespace tq {
namespace {

constexpr int kThreads = 256;

// round((v - zero) / scale) to nearest even, clamped to [0, levels].  The fp32
// quotient, (v - zero) times the group's rounded reciprocal of the scale, is
// within 4e-6 of the exact one (three roundings of 2^-24 relative, |q| <= 16),
// so it decides every case except those within 1e-4 of a half-integer, which
// are redone in fp64.
__device__ __forceinline__ uint32_t value_code(float v, float zero, float scale, float inv_scale, int levels)
{
    if (scale == 0.0f) return 0;
    float q = (v - zero) * inv_scale;
    const float frac = q - floorf(q);
    float r;
    if (fabsf(frac - 0.5f) < 1e-4f) {
        r = static_cast<float>(rint((static_cast<double>(v) - static_cast<double>(zero)) /
                                    static_cast<double>(scale)));
    } else {
        r = rintf(q);
    }
    r = fminf(fmaxf(r, 0.0f), static_cast<float>(levels));
    return static_cast<uint32_t>(r);
}

template <typename TIn, int G, int BITS>
__global__ __launch_bounds__(kThreads) void k_compress_values(ValueLaunch a, int64_t n_groups)
{
    const int64_t g0 = static_cast<int64_t>(blockIdx.x) * kThreads;   // workgroup-uniform
    const int64_t gi = g0 + threadIdx.x;
    if (gi >= n_groups) return;
    // groups per vector is a power of two dividing the workgroup size: one
    // divide per workgroup, then each thread steps from (b0, h0, t0)
    const int lg = __builtin_ctz(a.d / G);
    const int64_t nfirst = g0 >> lg;
    const int off = static_cast<int>(threadIdx.x) >> lg;
    const int grp = static_cast<int>(threadIdx.x) & ((1 << lg) - 1);
    const int64_t n = nfirst + off;
    const int64_t bh0 = nfirst / a.T;
    int64_t t = nfirst - bh0 * a.T + off;
    int64_t b = bh0 / a.H, h = bh0 - b * a.H;
    while (t >= a.T) {                  // at most kThreads / T + 1 steps
        t -= a.T;
        if (++h == a.H) {
            h = 0;
            ++b;
        }
    }
    const TIn *src = static_cast<const TIn *>(a.v) + b * a.sb + h * a.sh + t * a.st + grp * G;

    float x[G];
#pragma unroll
    for (int i = 0; i < G / 8; ++i) {
        float v8[8];
        load8_as_f32(src + 8 * i, v8);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * i + e] = v8[e];
    }
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < G; ++i) {
        mn = fminf(mn, x[i]);
        mx = fmaxf(mx, x[i]);
    }
    constexpr int levels = (1 << BITS) - 1;
    const uint32_t sh = f64_to_f16_rne((static_cast<double>(mx) - static_cast<double>(mn)) / levels);
    const uint32_t zh = f64_to_f16_rne(static_cast<double>(mn));
    const float sc = f16_bits_to_f32(sh), ze = f16_bits_to_f32(zh);
    const float inv = sc != 0.0f ? 1.0f / sc : 0.0f;

    constexpr int per_word = 32 / BITS, words = G * BITS / 32;
    const int64_t row = out_row(a.map, a.H, a.T, n);      // n itself unless appending
    if (row < 0) return;
    uint32_t *dst = reinterpret_cast<uint32_t *>(a.out.codes) + row * (a.d * BITS / 32) + grp * words;
#pragma unroll
    for (int w = 0; w < words; ++w) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < per_word; ++e)
            word |= value_code(x[w * per_word + e], ze, sc, inv, levels) << (BITS * e);
        dst[w] = word;
    }
    reinterpret_cast<uint32_t *>(a.out.params)[row * (a.d / G) + grp] = sh | (zh << 16);
}

template <typename TIn, int G, int BITS>
hipError_t launch_v(const ValueLaunch &a, hipStream_t stream)
{
    const int64_t n_groups = static_cast<int64_t>(a.B) * a.H * a.T * (a.d / G);
    const int64_t blocks = (n_groups + kThreads - 1) / kThreads;
    void *tok;
    prof_begin("tq_compress_values", stream, &tok);
    hipLaunchKernelGGL((k_compress_values<TIn, G, BITS>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, stream, a, n_groups);
    prof_end(tok, stream);
    return hipGetLastError();
}

template <typename TIn, int G>
hipError_t launch_vb(const ValueLaunch &a, hipStream_t stream)
{
    return a.bits == 2 ? launch_v<TIn, G, 2>(a, stream) : launch_v<TIn, G, 4>(a, stream);
}

template <typename TIn>
hipError_t launch_vg(const ValueLaunch &a, hipStream_t stream)
{
    switch (a.group) {
    case 32: return launch_vb<TIn, 32>(a, stream);
    case 64: return launch_vb<TIn, 64>(a, stream);
    case 128: return launch_vb<TIn, 128>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_compress_values(const ValueLaunch &a, hipStream_t stream)
{
    switch (a.dtype) {
    case TQ_F32: return launch_vg<float>(a, stream);
    case TQ_BF16: return launch_vg<bf16_t>(a, stream);
    case TQ_F16: return launch_vg<f16_t>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace tq
