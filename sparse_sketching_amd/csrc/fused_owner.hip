// Fused SparseStack sketch of narrow matrices by output-row owners, for
// gfx950.  Same sketch, same metadata and same arithmetic as the register
// kernel of fused.hip (FP16 sketching page §III-A, §III-B: FP32 products,
// in the FP16 variant each rounded to FP16 nearest-even and added with FP16
// nearest-even additions; metadata drawn in the kernel from Philox-4x32-10,
// §III-C, never stored, as on the FlashSketch page §5.2), and the same order
// of additions: every output entry adds the contributions of its workgroup's
// row chunk in ascending row order from +0, and the chunk partials are then
// summed by the fixed-order reduce.
//
// Why a second kernel: in the register kernel a wavefront keeps R output
// rows x one column slice, and every hit costs a ballot share, scalar
// bookkeeping and one LDS round trip for 64 lanes x W words.  For narrow rows
// most of those lanes are idle (a 64-column FP16 row fills half of them, a
// right-hand side of 2 columns one), while the per-hit cost stays.  Here the
// lanes own the output rows instead:
//  * A workgroup owns all d output rows of one chunk of input rows: lane
//    (o, g) keeps words [g*V, (g+1)*V) of output row o in registers (L = U/V
//    lanes per row, U = the row's words padded to a power of two).
//  * Rows stream through LDS in stages of S rows (two or three buffers).  For
//    each stage the kernel draws the Philox words of its rows, sets bit j of
//    a per-output-row hit mask for every hit (integer LDS atomic OR, order
//    free), then ranks each hit among the hits of its output row (the
//    popcount of the mask below j: a stable counting sort) and writes it to
//    that row's list.  Each lane then walks its row's list in ascending row
//    order, one packed FMA by +-1 per word and hit, with no scalar work per
//    hit: a wavefront serves 64/L output rows per list step.
//  * A list holds up to `cap` hits; an output row with more hits in a stage
//    walks the rest straight from its mask (same order, slower).
//  * Two barriers per stage, or one where the LDS holds a third stage
//    buffer, mask set and entry set at the same stage rows (then stage s is
//    walked, s + 1 ranked and s + 2 staged and drawn in one phase); the
//    next stages' rows are in flight from HBM meanwhile (loads with the
//    nontemporal hint: A is read once).
#include "sk_internal.hpp"
#include "sk_rng.hpp"
#include "sk_stack_apply.hpp"
#include "sk_stream.hpp"

namespace sk {
namespace {

struct OwnerArgs {
    const float *A;
    uint32_t *ws;               // [chunks][d][U] partial words
    int64_t m, lda, rows_per_chunk, row_offset;
    uint64_t seed;
    int32_t n_words;            // words of a row (columns, or column pairs for FP16)
    int32_t U, L;               // words per row padded to a power of two; lanes per output row
    int32_t d, zeta;
    int32_t S, cap;             // input rows per stage; list capacity per output row
    int32_t ms, cs;             // words between output rows' masks, lists
    float scale;                // float32(1/sqrt(zeta))
};

constexpr int kOwnerLoads = 4;          // loads per thread and stage (at most)
// words of an output row per lane (more would not fit the registers of a
// 1024-thread workgroup next to the staged loads)
constexpr int kOwnerMaxWords = 16;
// input rows per stage (at most)
constexpr int kOwnerMaxStage = 512;

// V words of LDS as one access (ds_read_b32/_b64/_b128 per 4 words)
template <int V>
__device__ __forceinline__ void read_words(const uint32_t *p, uint32_t (&x)[V]) {
    if constexpr (V == 1) {
        x[0] = p[0];
    } else if constexpr (V == 2) {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        x[0] = v.x;
        x[1] = v.y;
    } else {
#pragma unroll
        for (int i = 0; i < V; i += 4) {
            const uint4 v = *reinterpret_cast<const uint4 *>(p + i);
            x[i] = v.x;
            x[i + 1] = v.y;
            x[i + 2] = v.z;
            x[i + 3] = v.w;
        }
    }
}

// Words between consecutive output rows' mask (or list) words: at least w +
// 4 (the 4 count words after the mask; for a list, room for a 16-byte read
// at its last slot); where the LDS allows, an odd number of 16-byte units,
// so that 16 lanes reading consecutive rows' words at one offset hit 16
// distinct groups of 4 banks.
constexpr int owner_row_stride(int w, bool spread) {
    return (spread && ((w >> 2) & 1)) ? w + 8 : w + 4;
}

// The sign bits of T's +-1 word (FP16 pair: both halves)
template <class T> constexpr uint32_t kUnitSign = T::kCols == 2 ? 0x80008000u : 0x80000000u;

// OB: one barrier per stage (three stage buffers, mask and entry sets, two
// list sets); else two (two of each, one list set).  NL: load slots per
// thread and stage (kOwnerLoads, or 2 at 16 words per lane where a stage
// needs no more: its two register sets then fit without spilling)
template <class T, int V, int KF, bool OB, int NL>
__global__ __launch_bounds__(1024, 1) void k_stack_owner(const OwnerArgs args) {
    extern __shared__ __align__(16) uint32_t lds[];
    const int NT = (int)blockDim.x;
    const int NW = NT >> 6;
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int S = args.S, U = args.U, L = args.L, d = args.d, zeta = args.zeta;
    const int s_log = 31 - __builtin_clz((unsigned)S);
    const int u_log = 31 - __builtin_clz((unsigned)U);
    const int MW = S >> 5;              // mask words per output row (a multiple of 4)
    const int MS = args.ms;             // a row's mask words, then its 4 count words
    const int CS = args.cs;             // list stride in words
    const uint32_t cap = (uint32_t)args.cap;
    const uint32_t db = (uint32_t)(d / zeta);
    // LDS, in words (NB = 3 with one barrier per stage, else 2):
    //  * NB stage buffers [S + 1][U] (row S: the -0 row that unused list
    //    slots point at), padding to 16 bytes, 4 trash words;
    //  * NB mask sets [d][MS]: per output row, MW words of hit bits (bit j:
    //    stage row j hits the row), then per 64 stage rows a byte count of
    //    its hits (at most 8 bytes, in 4 words with the padding);
    //  * NB entry sets [zeta][S]: output row | sign << 31 of (block, row),
    //    ~0 for a row past the chunk;
    //  * NB - 1 list sets [d][CS]: per output row its hits in ascending row
    //    order, as the row's word offset in a stage buffer | unit sign bits.
    constexpr int NB = OB ? 3 : 2;
    const int BS = (S + 1) * U;
    uint32_t *const bufs = lds;
    const uint32_t trash = (uint32_t)((NB * BS + 3) & ~3);
    uint32_t *const masks = bufs + trash + 4;
    const int MSET = d * MS;            // words of a mask set
    uint32_t *const ents = masks + NB * MSET;
    const int ESET = zeta * S;          // words of an entry set
    uint32_t *const lsts = ents + NB * ESET;
    const int LSET = d * CS;            // words of a list set

    const int32_t chunk = blockIdx.x;
    const int64_t r0 = (int64_t)chunk * args.rows_per_chunk;
    const int32_t nrows =
        (int32_t)(r0 + args.rows_per_chunk < args.m ? args.rows_per_chunk : args.m - r0);
    const int32_t nst = (nrows + S - 1) / S;
    const float c = args.scale;
    constexpr int KC = T::kCols;

    // this thread's share of a stage's loads: load q = tid + i*NT covers
    // words [w0, w0 + KW) of stage row q / (U/KW); two sets of registers,
    // so two stages are in flight.  Every load is issued (rows past the
    // chunk and words past the row are clamped to valid memory; staging
    // drops them), so each set's registers are written by one load each.
    constexpr int KW = KF / KC;                     // words per load
    const int lpr_log = u_log - (KW == 4 ? 2 : KW == 2 ? 1 : 0);    // loads per row, log2
    const int nq = S << lpr_log;                    // loads of a stage
    const uint32_t lda4 = (uint32_t)args.lda * 4u;
    const char *const A = reinterpret_cast<const char *>(args.A);
    // the thread's load slots, the same for every stage: slot i is load
    // q = tid + i*NT of the stage (a thread with fewer loads than slots
    // repeats the stage's last load: one address, no new bytes), row lrow,
    // first float at byte lcol of the row; staged at word soff of a stage
    // buffer (the trash words for a repeated load), words past the row's
    // (padding) masked to zero
    uint32_t lrow[NL], lcol[NL], soff[NL], keep[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int q = tid + i * NT;
        const int qc = q < nq ? q : nq - 1;
        const int w0 = (qc & ((1 << lpr_log) - 1)) * KW;
        lrow[i] = (uint32_t)(qc >> lpr_log);
        lcol[i] = (uint32_t)((w0 < args.n_words ? w0 : 0) * KC * 4);
        soff[i] = q < nq ? (uint32_t)(((qc >> lpr_log) << u_log) + w0) : trash;
        keep[i] = w0 < args.n_words ? ~0u : 0u;
    }
    FVec<KF> ld[2][NL];
    auto load = [&](int32_t s, FVec<KF> (&dst)[NL]) {
        const int32_t first = s * S < nrows ? s * S : 0;
        const char *base = A + (r0 + first) * (int64_t)lda4;
        const uint32_t last = (uint32_t)(nrows - 1 - first);     // last valid row of the stage
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const uint32_t row = lrow[i] < last ? lrow[i] : last;
            dst[i] = load_vec<KF, true>(base + row * lda4 + lcol[i]);
        }
    };
    // the loaded rows' contribution words into stage buffer buf
    auto stage = [&](const FVec<KF> (&src)[NL], uint32_t *buf) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            uint32_t *dst = (soff[i] == trash ? bufs : buf) + soff[i];
            uint32_t w[KW];
#pragma unroll
            for (int k = 0; k < KW; ++k) w[k] = T::contrib(&src[i].x[k * KC], c) & keep[i];
            if constexpr (KW == 4)
                *reinterpret_cast<uint4 *>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
            else if constexpr (KW == 2)
                *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
            else
                dst[0] = w[0];
        }
    };
    // the hits of stage s: entries, mask bits and per-64-row counts (one
    // row per thread; integer LDS atomics, whose order does not matter)
    const uint32_t k0 = (uint32_t)args.seed, k1 = (uint32_t)(args.seed >> 32);
    auto draw = [&](int32_t s, uint32_t *mk, uint32_t *ent) {
        for (int j = tid; j < S; j += NT) {
            const bool valid = s * S + j < nrows;
            const uint64_t g = (uint64_t)args.row_offset + (uint64_t)(r0 + (int64_t)s * S + j);
            for (int gq = 0; gq * 4 < zeta; ++gq) {
                const u32x4 w4 = philox4x32_10(
                    u32x4{(uint32_t)g, (uint32_t)(g >> 32), (uint32_t)gq, 0u}, k0, k1);
                const uint32_t ww[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
                for (int jw = 0; jw < 4; ++jw) {
                    const int t = gq * 4 + jw;
                    if (t < zeta) {
                        const uint32_t o = (uint32_t)t * db + mulhi32(ww[jw], db);
                        ent[(t << s_log) + j] = valid ? (o | (ww[jw] << 31)) : 0xFFFFFFFFu;
                        if (valid) {
                            uint32_t *mo = mk + __umul24(o, (uint32_t)MS);
                            __hip_atomic_fetch_or(mo + (j >> 5), 1u << (j & 31), __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_WORKGROUP);
                            __hip_atomic_fetch_add(mo + MW + (j >> 8), 1u << (((j >> 6) & 3) * 8),
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                        }
                    }
                }
            }
        }
    };
    // every hit of a stage into its output row's list.  Its rank among its
    // row's hits: the row's hits in earlier 64-row groups (the group byte
    // counts below it) plus those before it in its own group (mbcnt of the
    // group's 64 mask bits: a wavefront takes one group of one block, lane =
    // row mod 64).  Two groups per pass, their reads issued together.
    auto rank = [&](const uint32_t *mk, const uint32_t *ent, uint32_t *lst) {
        const int per_t = S >> 6;
        const int groups = zeta * per_t;
        for (int g0 = wave; g0 < groups; g0 += 2 * NW) {
            int gi[2], jb[2];
            uint32_t e[2], o2[2];
            uint2 mw[2], cw[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                gi[h] = g0 + h * NW < groups ? g0 + h * NW : g0;
                const int t = gi[h] / per_t;
                jb[h] = gi[h] - t * per_t;
                e[h] = ent[(t << s_log) + jb[h] * 64 + lane];
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                o2[h] = e[h] != 0xFFFFFFFFu ? (e[h] & 0x7FFFFFFFu) : 0u;
                const uint32_t *mo = mk + __umul24(o2[h], (uint32_t)MS);
                mw[h] = *reinterpret_cast<const uint2 *>(mo + 2 * jb[h]);
                cw[h] = *reinterpret_cast<const uint2 *>(mo + MW);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (h == 1 && g0 + NW >= groups) break;
                // byte counts of the groups below jb (jb wave-uniform)
                const int b = jb[h];
                const uint32_t m0 = b >= 4 ? ~0u : (b == 0 ? 0u : (1u << (8 * b)) - 1u);
                const uint32_t m1 = b <= 4 ? 0u : (1u << (8 * (b - 4))) - 1u;
                uint32_t r = __builtin_amdgcn_sad_u8(cw[h].x & m0, 0u, 0u);
                r = __builtin_amdgcn_sad_u8(cw[h].y & m1, 0u, r);
                r = __builtin_amdgcn_mbcnt_hi(mw[h].y, __builtin_amdgcn_mbcnt_lo(mw[h].x, r));
                const int j = jb[h] * 64 + lane;
                if (e[h] != 0xFFFFFFFFu && r < cap)
                    lst[__umul24(o2[h], (uint32_t)CS) + r] =
                        ((uint32_t)j << u_log) | ((e[h] >> 31) ? kUnitSign<T> : 0u);
            }
        }
    };

    // the lane's output row and words
    const int o = tid / L;
    const int g = tid - o * L;
    const int t_o = o / (int)db;
    uint32_t acc[V];
#pragma unroll
    for (int k = 0; k < V; ++k) acc[k] = 0u;
    const uint32_t one = T::unit(0u);
    const uint32_t lane_w = (uint32_t)(g * V);      // the lane's first word of a row
    // one hit (list entry form: the row's word offset | unit sign bits) on
    // stage buffer buf
    auto hit = [&](const uint32_t *buf, uint32_t e) {
        const uint32_t *src = buf + lane_w + (e & 0x7FFFu);
        const uint32_t u = one | (e & kUnitSign<T>);
        constexpr int VC = V < 4 ? V : 4;       // words per LDS read
#pragma unroll
        for (int i = 0; i < V; i += VC) {
            uint32_t x[VC];
            read_words<VC>(src + i, x);
#pragma unroll
            for (int k = 0; k < VC; ++k) acc[i + k] = T::fma_unit(x[k], u, acc[i + k]);
        }
    };
    const uint32_t my_list_off = __umul24((uint32_t)o, (uint32_t)CS);
    const uint32_t my_mask = __umul24((uint32_t)o, (uint32_t)MS);
    // zero the lane's share of its row's mask and count words
    auto clear_row = [&](uint32_t *mk) {
        for (int q = g * 4; q < MS; q += L * 4)
            *reinterpret_cast<uint4 *>(mk + my_mask + q) = make_uint4(0u, 0u, 0u, 0u);
    };
    // stage s's hits of the lane's output row, in ascending row order; a
    // list slot past the row's hits points at the -0 row (x * +1 = -0 adds
    // nothing to any value), so list steps take no branches (below 16 words)
    const uint32_t dummy = (uint32_t)(S << u_log);
    auto walk = [&](const uint32_t *buf, uint32_t *mk, const uint32_t *ent,
                    const uint32_t *lst) -> bool {
        const uint32_t *const my_list = lst + my_list_off;
        const uint2 cw = *reinterpret_cast<const uint2 *>(mk + my_mask + MW);
        const uint32_t count = __builtin_amdgcn_sad_u8(cw.y, 0u, __builtin_amdgcn_sad_u8(cw.x, 0u, 0u));
        const uint32_t cnt = count < cap ? count : cap;
        // the row's count words are read (the L lanes of a row share a
        // wavefront, whose LDS accesses complete in order); clear its words
        // for the next stage that uses this mask set, each lane its share,
        // except where the rest of the row's hits are walked from the mask
        // below
        if (count <= cap) clear_row(mk);
        for (uint32_t p = 0; __ballot(p < cnt) != 0; p += 4) {
            const uint4 e4 = *reinterpret_cast<const uint4 *>(my_list + p);
            if constexpr (V >= 16) {
                // four LDS reads per hit: lanes past their row's count skip
                // them (masked) rather than read the -0 row, whose reads
                // would cost LDS bandwidth (7-13% faster at 16 words)
                if (p < cnt) hit(buf, e4.x);
                if (p + 1 < cnt) hit(buf, e4.y);
                if (p + 2 < cnt) hit(buf, e4.z);
                if (p + 3 < cnt) hit(buf, e4.w);
            } else {
                hit(buf, p < cnt ? e4.x : dummy);
                hit(buf, p + 1 < cnt ? e4.y : dummy);
                hit(buf, p + 2 < cnt ? e4.z : dummy);
                hit(buf, p + 3 < cnt ? e4.w : dummy);
            }
        }
        // more hits than the list holds: the rest from the mask, after the
        // list's last row
        if (__ballot(count > cap) != 0 && count > cap) {
            const uint32_t *mo = mk + my_mask;
            const uint32_t j0 = ((my_list[cap - 1] & 0x7FFFu) >> u_log) + 1;
            for (int q = (int)(j0 >> 5); q < MW; ++q) {
                uint32_t w = mo[q];
                if (q == (int)(j0 >> 5)) w &= ~0u << (j0 & 31);
                while (w != 0) {
                    const uint32_t j = (uint32_t)q * 32 + (uint32_t)__builtin_ctz(w);
                    w &= w - 1;
                    hit(buf, (j << u_log) | ((ent[(t_o << s_log) + j] >> 31) ? kUnitSign<T> : 0u));
                }
            }
        }
        return count > cap;
    };

    // masks and counts start clear; afterwards each row's words are cleared
    // once its stage is walked.  Row S of every stage buffer holds -0.
    for (int i = tid; i < NB * MSET; i += NT) masks[i] = 0u;
    for (int i = tid; i < U; i += NT)
#pragma unroll
        for (int k = 0; k < NB; ++k) bufs[k * BS + (S << u_log) + i] = kUnitSign<T>;
    __syncthreads();
    load(0, ld[0]);
    load(1, ld[1]);
    stage(ld[0], bufs);
    draw(0, masks, ents);
    load(2, ld[0]);
    if constexpr (OB) {
        if (1 < nst) {
            stage(ld[1], bufs + BS);
            draw(1, masks + MSET, ents + ESET);
        }
        load(3, ld[1]);
    }
    lds_barrier();
    rank(masks, ents, lsts);
    lds_barrier();
    if constexpr (OB) {
        // one barrier per stage: walk s, rank s + 1, stage and draw s + 2 in
        // one phase.  Stage buffers, mask and entry sets rotate over three
        // and list sets over two, so the sets a phase reads and writes are
        // disjoint: the walk reads (and clears its rows' masks in) set s
        // mod 3, the rank reads set s + 1 and writes list set s + 1 mod 2,
        // the draw writes set s + 2, which the previous phase walked and
        // cleared (before this phase's barrier-separated start).
        int32_t r3 = 0;                 // s mod 3
        for (int32_t s0 = 0; s0 < nst; s0 += 2) {
            // two stages per trip, so the register set index is a constant
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int32_t s = s0 + b;
                const int32_t i0 = r3, i1 = r3 == 2 ? 0 : r3 + 1, i2 = r3 == 0 ? 2 : r3 - 1;
                if (s < nst) {
                    uint32_t *mk = masks + i0 * MSET;
                    if (walk(bufs + i0 * BS, mk, ents + i0 * ESET, lsts + b * LSET))
                        clear_row(mk);
                }
                if (s + 1 < nst) rank(masks + i1 * MSET, ents + i1 * ESET, lsts + (b ^ 1) * LSET);
                // stage s + 2 from the set loaded two stages ago, then that
                // set takes stage s + 4 (issued on every path, clamped)
                if (s + 2 < nst) {
                    stage(ld[b], bufs + i2 * BS);
                    draw(s + 2, masks + i2 * MSET, ents + i2 * ESET);
                }
                load(s + 4, ld[b]);
                lds_barrier();
                r3 = i1;
            }
        }
    } else {
        for (int32_t s0 = 0; s0 < nst; s0 += 2) {
            // two stages per trip, so every buffer and register set index is
            // a constant; the loads are issued on every path (clamped past
            // the chunk), so each set's wait counts only the other set's loads
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int32_t s = s0 + b;
                const uint32_t *buf = bufs + b * BS, *ent = ents + b * ESET;
                uint32_t *mk = masks + b * MSET;
                uint32_t *buf1 = bufs + (b ^ 1) * BS, *mk1 = masks + (b ^ 1) * MSET,
                         *ent1 = ents + (b ^ 1) * ESET;
                // stage s+1 from the set loaded two stages ago, then that set
                // takes stage s+3
                if (s + 1 < nst) {
                    stage(ld[b ^ 1], buf1);
                    draw(s + 1, mk1, ent1);
                }
                load(s + 3, ld[b ^ 1]);
                // (a row walked past its list still needs its mask words
                // until the barrier; its lanes clear them after it)
                const bool over = s < nst && walk(buf, mk, ent, lsts);
                lds_barrier();
                if (s + 1 < nst) rank(mk1, ent1, lsts);
                if (over) clear_row(mk);
                lds_barrier();
            }
        }
    }
    // the loads past the last stage must land before exit
    __builtin_amdgcn_s_waitcnt(0);

    uint32_t *dst = args.ws + ((int64_t)chunk * d + o) * U + g * V;
    if constexpr (V >= 4) {
#pragma unroll
        for (int k = 0; k < V; k += 4)
            *reinterpret_cast<uint4 *>(dst + k) = make_uint4(acc[k], acc[k + 1], acc[k + 2], acc[k + 3]);
    } else if constexpr (V == 2) {
        *reinterpret_cast<uint2 *>(dst) = make_uint2(acc[0], acc[1]);
    } else {
        dst[0] = acc[0];
    }
}

template <class T, int KF, bool OB>
const void *pick_owner_v(int V, int nl) {
    if (nl == 2) return V == 16 ? (const void *)k_stack_owner<T, 16, KF, OB, 2> : nullptr;
    if (nl != kOwnerLoads) return nullptr;
    switch (V) {
    case 1: return (const void *)k_stack_owner<T, 1, KF, OB, kOwnerLoads>;
    case 2: return (const void *)k_stack_owner<T, 2, KF, OB, kOwnerLoads>;
    case 4: return (const void *)k_stack_owner<T, 4, KF, OB, kOwnerLoads>;
    case 8: return (const void *)k_stack_owner<T, 8, KF, OB, kOwnerLoads>;
    case 16: return (const void *)k_stack_owner<T, 16, KF, OB, kOwnerLoads>;
    default: return nullptr;
    }
}

// the built instances: FP16 loads of one or two words (2 or 4 floats), FP32
// of one or four; one or two barriers per stage; nl load slots
template <bool OB>
const void *pick_owner_b(bool f16, int V, int kw, int nl) {
    if (f16)
        return kw == 2 ? pick_owner_v<AccF16, 4, OB>(V, nl)
                       : kw == 1 ? pick_owner_v<AccF16, 2, OB>(V, nl) : nullptr;
    return kw == 4 ? pick_owner_v<AccF32, 4, OB>(V, nl)
                   : kw == 1 ? pick_owner_v<AccF32, 1, OB>(V, nl) : nullptr;
}
const void *pick_owner(bool f16, int V, int kw, int barriers, int nl) {
    return barriers == 1 ? pick_owner_b<true>(f16, V, kw, nl)
                         : barriers == 2 ? pick_owner_b<false>(f16, V, kw, nl) : nullptr;
}

}  // namespace

// nb: stage buffers, mask and entry sets (3: one barrier per stage, with two
// list sets; 2: two barriers, one list set)
size_t owner_lds_bytes(int32_t S, int32_t U, int32_t d, int32_t zeta, int32_t cap, bool spread,
                       int nb) {
    const size_t bufs = (size_t)nb * (S + 1) * U;
    return 4 * (((bufs + 3) & ~(size_t)3) + 4 + (size_t)nb * d * owner_row_stride(S / 32, spread) +
                (size_t)nb * zeta * S + (size_t)(nb - 1) * d * owner_row_stride(cap, spread));
}

// Plan of the owner kernel: FP16 rows of at most 64 column pairs, FP32 rows
// of at most 64 columns, whose d x U words fit one workgroup's registers at
// no more than kOwnerMaxWords words per lane.  Stage rows S (a multiple of 128) aim at
// about 8 hits per output row and stage (ranking balance) within the
// device's LDS and four loads per thread.
bool plan_owner(const DevInfo &di, bool f16, int64_t m, int32_t n, int64_t lda, int a_align,
                int32_t d, int32_t zeta, FusedPlan *p) {
    const int kc = f16 ? 2 : 1;
    if (m < 1 || n < kc || n % kc != 0 || zeta < 1 || zeta > kFusedMaxZeta || d % zeta != 0)
        return false;
    if (m > (int64_t)65535 << 30) return false;
    const int nw = n / kc;
    int U = 1;
    while (U < nw) U *= 2;
    if (U > 64) return false;
    // a one-word row at d <= 256 is padded to two words: twice the lanes and
    // wavefronts per CU for the same list walks (2^20 x 2 FP16 at d = 256:
    // 44 -> 38 us; at d = 512, 1024 threads instead of 512 were no faster)
    if (U == 1 && d <= 256) U = 2;
    // words per lane: the fewest with d x (U / V) <= 1024 threads, and whole
    // wavefronts
    int V = 1;
    while (V < U && (int64_t)d * (U / V) > 1024) V *= 2;
    if (V > kOwnerMaxWords) return false;
    int L = U / V;
    while ((d * L) % 64 != 0 && V > 1) {
        V /= 2;
        L *= 2;
    }
    const int64_t NT = (int64_t)d * L;
    if (NT > 1024 || NT % 64 != 0) return false;
    // words per load: FP16 two (16 bytes) or one; FP32 four or one
    int kw = 1;
    const int kmax = f16 ? 2 : 4;
    if (nw % kmax == 0 && U % kmax == 0 && lda % (kmax * kc) == 0 && a_align >= kmax * kc * 4)
        kw = kmax;
    if (kw == 1 && (lda % kc != 0 || a_align < kc * 4)) return false;
    // a stage's rows are addressed with 32-bit offsets from its first row
    if ((int64_t)kOwnerMaxStage * lda * 4 >= ((int64_t)1 << 31)) return false;
    // stage rows: ~8 hits per output row and stage, at most kOwnerLoads loads
    // per thread, at least 128 (a multiple of 128)
    int64_t S = 128;
    while (S * zeta < 8 * (int64_t)d && S < kOwnerMaxStage) S *= 2;
    while (S > 128 && S * U > (int64_t)kOwnerLoads * kw * NT) S /= 2;
    if (S * U > (int64_t)kOwnerLoads * kw * NT) return false;
    // list capacity: the mean hits per output row and stage plus two
    // standard deviations and two, in whole quads; the rare row with more
    // walks the rest from its mask
    auto cap_for = [&](int64_t s) {
        const double mu = (double)s * zeta / d;
        int64_t c = (int64_t)(mu + 2.0 * sqrt(mu) + 2.0 + 3.0) & ~(int64_t)3;
        if (c < 4) c = 4;
        if (c > s) c = s;
        return (int32_t)c;
    };
    while (S > 128 &&
           owner_lds_bytes((int32_t)S, U, d, zeta, cap_for(S), false, 2) > (size_t)di.max_lds)
        S /= 2;
    const int32_t cap = cap_for(S);
    const bool spread = owner_lds_bytes((int32_t)S, U, d, zeta, cap, true, 2) <= (size_t)di.max_lds;
    size_t lds = owner_lds_bytes((int32_t)S, U, d, zeta, cap, spread, 2);
    if (lds > (size_t)di.max_lds) return false;
    auto per_cu_for = [&](size_t b) { return (size_t)di.max_lds >= 2 * b && NT <= 512 ? 2 : 1; };
    const int per_cu = per_cu_for(lds);
    // one barrier per stage where a third stage buffer, mask and entry set
    // and a second list set fit at the same stage rows and workgroups per
    // CU, for workgroups of 512 threads or more whose output rows average
    // at least 8 hits a stage (4 x 2^20 x 64 FP16 at d = 128: 226 -> 216
    // us, 2^20 x 32 FP16 at d = 256, zeta = 8: 72 -> 69 us; with fewer
    // threads or hits, as at 4 x 2^20 x 2 with d <= 128 or 2^20 x 128 FP16
    // at d = 128, zeta = 4, it ran up to 5% slower, and where it would need
    // fewer stage rows, slower still)
    const size_t lds1 = owner_lds_bytes((int32_t)S, U, d, zeta, cap, spread, 3);
    const bool one_barrier = NT >= 512 && S * zeta >= 8 * (int64_t)d &&
                             lds1 <= (size_t)di.max_lds && per_cu_for(lds1) == per_cu;
    if (one_barrier) lds = lds1;
    const int64_t stages = (m + S - 1) / S;
    int64_t want = (int64_t)di.num_cu * per_cu;
    if (want > stages) want = stages;
    if (want > 65535) want = 65535;
    const int64_t st_per_chunk = (stages + want - 1) / want;
    p->kind = kFusedOwner;
    p->words = V;
    p->dual = per_cu == 2 ? 1 : 0;
    p->stage_rows = (int)S;
    p->rows_per_wave = 64 / L;          // output rows a wavefront serves per list step
    p->groups = 1;
    p->load_sets = 1;
    p->slices = 1;
    p->rows_per_chunk = st_per_chunk * S;
    p->chunks = (m + p->rows_per_chunk - 1) / p->rows_per_chunk;
    p->grid = p->chunks;
    p->threads = (int)NT;
    p->row_words = U;
    p->lanes_per_row = L;
    p->cap = cap;
    p->mask_stride = owner_row_stride((int)S / 32, spread);
    p->list_stride = owner_row_stride(cap, spread);
    p->load_words = kw;
    p->lds_bytes = lds;
    p->barriers = one_barrier ? 1 : 2;
    // two load slots at 16 words per lane where a stage needs no more (four
    // spill: 2^20 x 32 FP16 at d = 1024, 108 -> 101 us; halving the stage
    // rows to fit two slots was slower: 2^20 x 64 FP16 at d = 512, 85 -> 97)
    p->load_slots = V == kOwnerMaxWords && S * U <= (int64_t)2 * kw * NT ? 2 : kOwnerLoads;
    p->ws_bytes = (size_t)p->chunks * (size_t)d * (size_t)U * 4;
    return true;
}

hipError_t launch_owner(const FusedPlan &p, bool f16, const float *A, int64_t m, int32_t n,
                        int64_t lda, uint64_t seed, int64_t row_offset, int32_t d, int32_t zeta,
                        float scale, void *B, int64_t ldb, uint32_t *ws, int mode,
                        hipStream_t s) {
    if (p.kind != kFusedOwner || ws == nullptr || (int64_t)p.threads != (int64_t)d * p.lanes_per_row)
        return hipErrorInvalidValue;
    OwnerArgs a{};
    a.A = A;
    a.ws = ws;
    a.m = m;
    a.lda = lda;
    a.rows_per_chunk = p.rows_per_chunk;
    a.row_offset = row_offset;
    a.seed = seed;
    a.n_words = f16 ? n / 2 : n;
    a.U = p.row_words;
    a.L = p.lanes_per_row;
    a.d = d;
    a.zeta = zeta;
    a.S = p.stage_rows;
    a.cap = p.cap;
    a.ms = p.mask_stride;
    a.cs = p.list_stride;
    a.scale = scale;
    // the load slots must cover a stage
    if ((int64_t)p.stage_rows * p.row_words > (int64_t)p.load_slots * p.load_words * p.threads)
        return hipErrorInvalidValue;
    const void *kern = pick_owner(f16, p.words, p.load_words, p.barriers, p.load_slots);
    if (kern == nullptr) return hipErrorInvalidValue;
    hipError_t e = set_lds_limit(kern, p.lds_bytes);
    if (e != hipSuccess) return e;
    void *params[] = {&a};
    e = hipLaunchKernel(kern, dim3((unsigned)p.grid), dim3((unsigned)p.threads), params,
                        p.lds_bytes, s);
    if (e != hipSuccess) return e;
    StackApplyArgs r{};
    r.B = B;
    r.ws = ws;
    r.ldb = f16 ? ldb / 2 : ldb;
    r.units = a.n_words;
    r.d = d;
    r.chunks = (int32_t)p.chunks;
    r.slices = 1;
    return f16 ? launch_stack_reduce<AccF16>(r, p.row_words, mode, s)
               : launch_stack_reduce<AccF32>(r, p.row_words, mode, s);
}

}  // namespace sk
