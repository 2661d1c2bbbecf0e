// Device-side tile movement shared by the matrix-core kernels (gfx950): global -> LDS
// copies (the LDS-DMA path of buffer and global loads) and transposed fragment reads of
// row-major tiles in LDS.  Index arithmetic lives in ssd_index.h.
#pragma once

#include "ssd_index.h"

namespace ssd {

// Raw LDS pointers for the gfx950 LDS-DMA and transpose-read builtins.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

// 16-byte global -> LDS copy: lane l of the wave writes lds_base + 16 * l.  The copies
// carry the non-temporal cache policy: every stream the kernels read this way is used once
// per step (measured: the whole step is ~4% faster with the streams marked so).
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ void dma16(const void *g, void *lds_base) {
    __builtin_amdgcn_global_load_lds(g, (lds_void_t *)lds_base, 16, 0, kCachePolicyNT);
}

// The per-head copies and stores go through buffer descriptors: a uniform base in scalar
// registers (rebuilt per head with scalar arithmetic) and a 32-bit per-lane offset, so a
// lane's address costs one vector register instead of two.  Offsets at or past `bytes`
// read zeros and drop stores (a bound on top of the kernels' own guards).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRawBufferWord3 = 0x00020000;     // untyped buffer, 32-bit data format (gfx9 family)
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRawBufferWord3);
}
__device__ __forceinline__ void dma16_buf(rsrc_t r, uint32_t voff, void *lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds_base, 16, voff, 0, 0, kCachePolicyNT);
}

// Fragment of a row-major [rows][W] tile in LDS (W elements per row; bf16 rows swizzled by
// x_swz in 16-byte pieces, fp32 rows plain) for (16-row block J, 16-column tile ct):
// lane (col, g) gets M[16J + 4g + e][16ct + col], e = 0..3 -- the operand layout of the
// contraction over rows (k = 4g + e of a K = 16 slice).  bf16: one gfx950 transpose read
// (ds_read_b64_tr_b16; lane s of a 16-lane group reads 4 columns of row 4g + s / 4);
// fp32: four scalar reads.
template <typename T, int W>
__device__ __forceinline__ typename TF<T>::type tile_frag(const unsigned char *m, int J, int ct, int lane) {
    if constexpr (sizeof(T) == 2) {
        return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t *)(m + tile_frag_read(J, ct, lane, W).off));
    } else {
        const int col = lane & 15, g = lane >> 4;
        const float *base = reinterpret_cast<const float *>(m) + (J * 16 + 4 * g) * W + ct * 16 + col;
        f32x4 v;
        v[0] = base[0];
        v[1] = base[W];
        v[2] = base[2 * W];
        v[3] = base[3 * W];
        return v;
    }
}

}  // namespace ssd
