// Device helpers for libtq kernels: storage types, vector loads, bit packing
// and exact fp16 rounding.
#pragma once

#include <hip/hip_runtime.h>

#include "tq_internal.h"

#include <cstdint>

namespace tq {

struct bf16_t { uint16_t bits; };
struct f16_t { uint16_t bits; };

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h)
{
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// eight consecutive elements (16-byte aligned for 2-byte types, 32-byte for fp32)
__device__ __forceinline__ void load8_as_f32(const float *p, float (&v)[8])
{
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void load8_as_f32(const bf16_t *p, float (&v)[8])
{
    const uint4 w = *reinterpret_cast<const uint4 *>(p);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_to_f32(u[i] & 0xffffu);
        v[2 * i + 1] = bf16_to_f32(u[i] >> 16);
    }
}

__device__ __forceinline__ void load8_as_f32(const f16_t *p, float (&v)[8])
{
    const uint4 w = *reinterpret_cast<const uint4 *>(p);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = f16_bits_to_f32(u[i] & 0xffffu);
        v[2 * i + 1] = f16_bits_to_f32(u[i] >> 16);
    }
}

// Word w of an LSB-first bit-stream whose element j (width `bits`) is vals[j].
__device__ __forceinline__ uint32_t pack_word(const uint8_t *vals, int w, int bits)
{
    const int first = (32 * w) / bits, last = (32 * w + 31) / bits;
    uint32_t word = 0;
    for (int j = first; j <= last; ++j) {
        const int off = bits * j - 32 * w;
        const uint32_t v = vals[j];
        word |= (off >= 0) ? (v << off) : (v >> (-off));
    }
    return word;
}

// IEEE binary16 bits of a double, round to nearest even (direct, no detour
// through fp32, so no double rounding).
__device__ __forceinline__ uint32_t f64_to_f16_rne(double x)
{
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
    const uint32_t sign = static_cast<uint32_t>(u >> 48) & 0x8000u;
    const uint64_t mag = u & 0x7fffffffffffffffULL;
    if (mag >= 0x7ff0000000000000ULL) return sign | (mag > 0x7ff0000000000000ULL ? 0x7e00u : 0x7c00u);
    const int e = static_cast<int>(mag >> 52) - 1023;
    if (e >= 16) return sign | 0x7c00u;
    if (e < -26) return sign;                      // below half the smallest subnormal
    const uint64_t sig = (mag & 0xfffffffffffffULL) | (1ULL << 52);   // normal doubles only here
    const int eh = e < -14 ? -14 : e;              // exponent of the fp16 ulp grid
    const int shift = 42 + (eh - e);               // sig * 2^(e-52) / 2^(eh-10)
    uint64_t q = sig >> shift;
    const uint64_t rem = sig & ((1ULL << shift) - 1), half = 1ULL << (shift - 1);
    if (rem > half || (rem == half && (q & 1))) ++q;
    if (e < -14) return sign | static_cast<uint32_t>(q);          // subnormal (q = 1024 -> min normal)
    return sign | (static_cast<uint32_t>(e + 15) << 10) + static_cast<uint32_t>(q) - 1024u;
}

// ---- layout caches (CacheMap): every index is checked, so that no access
// leaves the planes whatever the device tables hold

// row of token t of (b, h) in a layout cache, -1 outside it
__device__ __forceinline__ int64_t layout_row(const CacheMap &m, int H, int64_t b, int64_t h, int64_t t)
{
    if (t < 0 || t >= m.cap) return -1;
    if (m.mode == CacheMap::kContig) return (b * H + h) * m.cap + t;
    const int64_t blk = m.bt[b * m.maxb + t / m.bs];
    if (blk < 0 || blk >= m.nblocks) return -1;
    return (blk * H + h) * m.bs + t % m.bs;
}

// plane row of row n of a compress call over [B, H, T] inputs, -1 to skip
__device__ __forceinline__ int64_t out_row(const CacheMap &m, int H, int64_t T, int64_t n)
{
    if (m.mode == CacheMap::kFlat) return n;
    const int64_t t = n % T, bh = n / T;
    const int64_t b = bh / H, h = bh - b * H;
    return layout_row(m, H, b, h, static_cast<int64_t>(m.pos[b]) + t);
}

// tokens sequence b attends (T for a flat call)
__device__ __forceinline__ int64_t seq_len_of(const CacheMap &m, int64_t T, int64_t b)
{
    if (m.mode == CacheMap::kFlat) return T;
    const int64_t l = m.seq_lens[b];
    return l < 0 ? 0 : (l > m.cap ? m.cap : l);
}

}  // namespace tq
