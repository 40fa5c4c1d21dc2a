// Counter-based randomness shared by the host dispatch code and the gfx950
// kernels of libsksketch.
//
// * Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
//   as easy as 1, 2, 3", SC'11): a ten-round keyed bijection on 128-bit
//   counters.  One round multiplies counter words 0 and 2 by M0 and M1,
//   keeps both halves of each 64-bit product, and outputs
//   (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)); the key
//   is bumped by the Weyl constants between rounds.  The FP16 sketching
//   page (§III-C) names a coupled Philox kernel as the metadata source.
// * fmix32, the 32-bit finalizer of MurmurHash3 (Appleby): the "fast 32-bit
//   mixing hash" that the FlashSketch page (App. D, within-block hashing)
//   uses to route and sign rows on the fly.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define SK_HD __host__ __device__ __forceinline__
#else
#define SK_HD inline
#endif

namespace sk {

struct u32x4 {
    uint32_t x, y, z, w;
};

SK_HD u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
        c = u32x4{(uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1,
                  (uint32_t)(p0 >> 32) ^ c.w ^ k1, (uint32_t)p0};
    }
    return c;
}

SK_HD uint32_t mulhi32(uint32_t a, uint32_t b) {
    return (uint32_t)(((uint64_t)a * b) >> 32);
}

SK_HD uint32_t fmix32(uint32_t h) {
    h ^= h >> 16;
    h *= 0x85EBCA6Bu;
    h ^= h >> 13;
    h *= 0xC2B2AE35u;
    h ^= h >> 16;
    return h;
}

// Chained combine used to key the within-block hash by (seed, g, h).
SK_HD uint32_t hash_combine(uint32_t h, uint32_t x) {
    return fmix32(h ^ x) + 0x9E3779B9u;
}

SK_HD uint32_t blockperm_key(uint64_t seed, uint32_t g, uint32_t h) {
    uint32_t k = hash_combine(0x9E3779B9u, (uint32_t)seed);
    k = hash_combine(k, (uint32_t)(seed >> 32));
    k = hash_combine(k, g);
    return hash_combine(k, h);
}

}  // namespace sk
