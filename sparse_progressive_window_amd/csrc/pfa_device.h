// Device helpers shared by the PFA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pfa {

constexpr int kWave = 64;

// Window geometry of one layer call.
struct Geom {
    int B, heads, H, W, d;
    int win;     // 0 = global mode
    int shift;
    int N;       // tokens per window
    int nwy, nwx;
    int win_magic;  // ceil(65536 / win): t / win == (t * win_magic) >> 16 for t < 1024, win <= 32
};

// Pixel (raster index inside the head's H x W plane) of slot t of window (wy, wx):
// ((wy*win + t/win + shift) mod H, (wx*win + t%win + shift) mod W). The cyclic
// shift is an index remap; data never moves.
__device__ __forceinline__ int slot_pixel(const Geom& g, int wy, int wx, int t) {
    if (g.win == 0) return t;
    const int ty = (t * g.win_magic) >> 16;
    const int tx = t - ty * g.win;
    int y = wy * g.win + ty + g.shift;
    int x = wx * g.win + tx + g.shift;
    if (y >= g.H) y -= g.H;
    if (x >= g.W) x -= g.W;
    return y * g.W + x;
}

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }

// acc + a.lo * b.lo + a.hi * b.hi for two packed bf16 pairs (v_dot2c_f32_bf16: the
// bf16 products are exact in fp32, the sum accumulates in fp32)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), acc,
                                           false);
}

// Round to nearest even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
    uint32_t b = __float_as_uint(x);
    b += 0x7FFFu + ((b >> 16) & 1u);
    return b >> 16;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }
__device__ __forceinline__ int popc(uint64_t m) { return __builtin_popcountll(m); }
// Number of set bits of m below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Buffer resource over `bytes` bytes at `base` (raw, 32-bit elements); accesses
// past the end are dropped by the hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

}  // namespace pfa
