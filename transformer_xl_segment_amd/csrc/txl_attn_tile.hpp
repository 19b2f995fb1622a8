// txl_attn_tile.hpp -- register and LDS tile helpers shared by the attention
// kernels (forward and backward), on top of the MFMA layout of txl_device.hpp.
#pragma once

#include "txl_device.hpp"

namespace txl {

constexpr int kGPitch = 100;      // floats per query row of a distance buffer

// Two groups of four consecutive keys of one V^T row: keys [k0, k0+4) and [k0+8, k0+12).
__device__ __forceinline__ void load_vt(Frag<bf16> &f, const char *row, int k0) {
    bf16x4 lo = *reinterpret_cast<const bf16x4 *>(row + k0 * 2);
    bf16x4 hi = *reinterpret_cast<const bf16x4 *>(row + (k0 + 8) * 2);
    f.v = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ void load_vt(Frag<float> &f, const char *row, int k0) {
    f.lo = *reinterpret_cast<const f32x4 *>(row + k0 * 4);
    f.hi = *reinterpret_cast<const f32x4 *>(row + (k0 + 8) * 4);
}

// Registers [r0, r0+8) of an S^T block as the B operand of P.V.
__device__ __forceinline__ void p_frag(Frag<bf16> &f, const f32x16 &s, int r0) {
#pragma unroll
    for (int q = 0; q < 8; ++q) f.v[q] = (bf16)s[r0 + q];
}
__device__ __forceinline__ void p_frag(Frag<float> &f, const f32x16 &s, int r0) {
    f.lo = f32x4{s[r0], s[r0 + 1], s[r0 + 2], s[r0 + 3]};
    f.hi = f32x4{s[r0 + 4], s[r0 + 5], s[r0 + 6], s[r0 + 7]};
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Write one 32-distance block of G to the wave's distance buffer: register i of
// lane (a, hf) holds band offset e0 + crow(i), stored at position e0 + crow(i)
// of row a, so each group of four registers is one aligned 16-byte store.
__device__ __forceinline__ void write_gblock(float *grow, const f32x16 &g, int e0, int hf) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4 *>(grow + e0 + 8 * q + 4 * hf) = f32x4{g[4 * q], g[4 * q + 1], g[4 * q + 2], g[4 * q + 3]};
}

}  // namespace txl
