// Device helpers shared by the BlockPerm-SJLT kernels that work per input
// block (FlashSketch page §4 wiring, App. D affine full-cycle wiring).
#pragma once
#include "sk_internal.hpp"

namespace sk {

__device__ __forceinline__ uint32_t mod_mul(uint32_t x, uint32_t y, uint32_t M) {
    return (uint32_t)(((uint64_t)x * y) % M);
}

// The l-th reader of input block h (0 <= l < kappa): the output block g
// whose l-th neighbour is h.
__device__ __forceinline__ uint32_t bp_reader(const BlockPermGenArgs &a,
                                              const BlockPermTable &ginv, uint32_t h, int l) {
    if (a.wiring == 0) {
        // shift: pi_l(g) = (sigma(g) + l C) mod M, so g = sigma^-1(h - l C)
        const uint32_t M = (uint32_t)a.M;
        const uint32_t x = (h + M - (uint32_t)((int64_t)l * a.C % M)) % M;
        return ginv.tab[x];
    }
    // affine: pi_l = f^(l+1), so g = f^-(l+1)(h), f^-1(x) = a^-1 (x - b)
    uint32_t x = h;
    for (int i = 0; i <= l; ++i)
        x = mod_mul(a.ainv, (x + (uint32_t)a.M - a.b) % (uint32_t)a.M, (uint32_t)a.M);
    return x;
}

}  // namespace sk
