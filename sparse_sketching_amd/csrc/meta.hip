// SparseStack metadata generation and output zeroing on gfx950.
//
// Metadata (FP16 sketching page §III-C): one Philox-4x32-10 block per
// (global row, group of four stack blocks); stack block t routes with word
// t mod 4 (multiply-high bucket, bit-0 sign).  One thread makes one block
// and writes up to four (row_idx, val) entries; when zeta is a multiple of
// four and the arrays are 16-byte aligned it writes them as one 16-byte
// store each, so a wavefront writes 1 KiB of contiguous metadata per store.
// The stores carry the nontemporal hint: the apply that reads the arrays
// next ran 15 % slower (0.246 against 0.209 ms for metadata + register
// apply of a 2^20 x 256 matrix on gfx950) when they were cached writes.
#include "sk_internal.hpp"
#include "sk_rng.hpp"

namespace sk {
namespace {

template <bool VEC4>
__global__ __launch_bounds__(256) void k_meta(uint64_t seed, int64_t row_offset, int64_t m,
                                              int32_t zeta, int32_t ngroups, uint32_t db,
                                              float scale, int32_t *__restrict__ row_idx,
                                              float *__restrict__ val) {
    const int64_t total = m * ngroups;
    for (int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x; tid < total;
         tid += (int64_t)gridDim.x * 256) {
    const int64_t i = ngroups == 1 ? tid : tid / ngroups;
    const int32_t grp = (int32_t)(tid - i * ngroups);
    const uint64_t g = (uint64_t)row_offset + (uint64_t)i;
    const u32x4 w = philox4x32_10(u32x4{(uint32_t)g, (uint32_t)(g >> 32), (uint32_t)grp, 0u},
                                  (uint32_t)seed, (uint32_t)(seed >> 32));
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    const int32_t t0 = grp * 4;
    const int64_t e = i * zeta + t0;
    int32_t r[4];
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        r[j] = (int32_t)((uint32_t)(t0 + j) * db + mulhi32(ws[j], db));
        v[j] = (ws[j] & 1u) ? -scale : scale;
    }
    if (VEC4) {
        typedef int i4_t __attribute__((ext_vector_type(4)));
        typedef float f4_t __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(i4_t{r[0], r[1], r[2], r[3]},
                                    reinterpret_cast<i4_t *>(row_idx + e));
        __builtin_nontemporal_store(f4_t{v[0], v[1], v[2], v[3]},
                                    reinterpret_cast<f4_t *>(val + e));
    } else {
        const int32_t cnt = zeta - t0 < 4 ? zeta - t0 : 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < cnt) {
                __builtin_nontemporal_store(r[j], row_idx + e + j);
                __builtin_nontemporal_store(v[j], val + e + j);
            }
        }
    }
    }
}

__global__ __launch_bounds__(256) void k_zero_words(uint32_t *__restrict__ B, int64_t rows,
                                                    int64_t words, int64_t ld_words) {
    const int64_t total = rows * words;
    for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < total;
         k += (int64_t)gridDim.x * 256) {
        const int64_t r = k / words;
        B[r * ld_words + (k - r * words)] = 0u;
    }
}

}  // namespace

hipError_t launch_meta(uint64_t seed, int64_t row_offset, int64_t m, int32_t d, int32_t zeta,
                       float scale, int32_t *row_idx, float *val, hipStream_t stream) {
    const int32_t ngroups = (zeta + 3) / 4;
    const uint32_t db = (uint32_t)(d / zeta);
    const int64_t threads = m * ngroups;
    int64_t blocks = (threads + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;
    const dim3 grid((unsigned)blocks);
    const bool vec4 = (zeta % 4 == 0) && ((uintptr_t)row_idx % 16 == 0) &&
                      ((uintptr_t)val % 16 == 0);
    if (vec4)
        k_meta<true><<<grid, 256, 0, stream>>>(seed, row_offset, m, zeta, ngroups, db, scale,
                                               row_idx, val);
    else
        k_meta<false><<<grid, 256, 0, stream>>>(seed, row_offset, m, zeta, ngroups, db, scale,
                                                row_idx, val);
    return hipGetLastError();
}

hipError_t launch_zero_words(uint32_t *B, int64_t rows, int64_t words, int64_t ld_words,
                             hipStream_t stream) {
    const int64_t total = rows * words;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    k_zero_words<<<dim3((unsigned)blocks), 256, 0, stream>>>(B, rows, words, ld_words);
    return hipGetLastError();
}

}  // namespace sk
