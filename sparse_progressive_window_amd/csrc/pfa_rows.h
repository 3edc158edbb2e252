// Row-level helpers shared by the window-mode kernels (gfx950, wave64):
// DPP lane exchanges, 16-byte chunk unpacking, workgroup -> window-head
// decoding and LDS staging of a window's rows.
#pragma once

#include "pfa_device.h"

namespace pfa {

// DPP controls (GFX9 encoding)
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowRor2 = 0x122;
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7 - i inside each 8-lane half-row

template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __int_as_float(dpp<CTRL>(__float_as_int(v)));
}
__device__ __forceinline__ int swap16(int v) { return __builtin_amdgcn_ds_swizzle(v, 0x401F); }
__device__ __forceinline__ float swap16f(float v) { return __int_as_float(swap16(__float_as_int(v))); }

template <typename T>
struct Chunk;

template <>
struct Chunk<float> {
    static constexpr int kElems = 4;
    __device__ static void to_f32(const uint4 c, float* o) {
        o[0] = __uint_as_float(c.x);
        o[1] = __uint_as_float(c.y);
        o[2] = __uint_as_float(c.z);
        o[3] = __uint_as_float(c.w);
    }
};

template <>
struct Chunk<uint16_t> {  // bf16 bit patterns
    static constexpr int kElems = 8;
    __device__ static void to_f32(const uint4 c, float* o) {
        o[0] = bf16_lo(c.x); o[1] = bf16_hi(c.x);
        o[2] = bf16_lo(c.y); o[3] = bf16_hi(c.y);
        o[4] = bf16_lo(c.z); o[5] = bf16_hi(c.z);
        o[6] = bf16_lo(c.w); o[7] = bf16_hi(c.w);
    }
};

struct WhPart {
    int wh, part, wy, wx, b, bh, win_id, nwin;
};

// window coordinates of window-head wh
__device__ __forceinline__ WhPart wh_coords(int wh, int part, const Geom& g) {
    WhPart w;
    w.wh = wh;
    w.part = part;
    w.nwin = g.nwy * g.nwx;
    w.win_id = w.wh % w.nwin;
    w.bh = w.wh / w.nwin;
    w.b = w.bh / g.heads;
    w.wy = w.win_id / g.nwx;
    w.wx = w.win_id - w.wy * g.nwx;
    return w;
}

// workgroup -> (window-head, part); with xcd_map the parts of one window-head are
// consecutive workgroups of one XCD (workgroups are dealt to the 8 XCDs in turn)
__device__ __forceinline__ WhPart decode_block_id(int bid, int blocks_per_wh, int xcd_map, const Geom& g) {
    WhPart w;
    if (xcd_map) {
        const int xcd = bid & 7;
        const int slot = bid >> 3;
        w.part = slot % blocks_per_wh;
        w.wh = (slot / blocks_per_wh) * 8 + xcd;
    } else {
        w.wh = bid / blocks_per_wh;
        w.part = bid - w.wh * blocks_per_wh;
    }
    w.nwin = g.nwy * g.nwx;
    w.win_id = w.wh % w.nwin;
    w.bh = w.wh / w.nwin;
    w.b = w.bh / g.heads;
    w.wy = w.win_id / g.nwx;
    w.wx = w.win_id - w.wy * g.nwx;
    return w;
}
__device__ __forceinline__ WhPart decode_block(int blocks_per_wh, int xcd_map, const Geom& g) {
    return decode_block_id(blockIdx.x, blocks_per_wh, xcd_map, g);
}

// Stage rows t = 0..N-1 of a window (slot order, under the layer's shift) into LDS
// with a row stride of `stride` bytes.
template <typename T, int D>
__device__ __forceinline__ void stage_rows(unsigned char* dst, int stride, const T* src_plane, const Geom& g, int wy,
                                           int wx) {
    constexpr int EPC = Chunk<T>::kElems;
    constexpr int CH = D / EPC;
    for (int u = threadIdx.x; u < g.N * CH; u += blockDim.x) {
        const int t = u / CH;
        const int c = u - t * CH;
        const size_t src = (size_t)slot_pixel(g, wy, wx, t) * D + c * EPC;
        *reinterpret_cast<uint4*>(dst + t * stride + c * 16) = *reinterpret_cast<const uint4*>(src_plane + src);
    }
}


}  // namespace pfa
