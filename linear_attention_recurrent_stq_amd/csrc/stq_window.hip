// Windowed decode for gfx950 (LeapQuant article, "研究の概要": the low-bit
// state is requantized only at the end of a window of W tokens; inside the
// window outputs come from the fixed low-bit base plus updates kept in high
// precision; large outliers are kept as a few high-precision "compensation"
// entries that ride the ordinary update path).
//
// Per state and step, with n deltas stored (cumulative gate g, deltas
// (u_m, kap_m) for m < n, base B = RN(n_ij r_i c_j), compensation entries
// (p = j*d_k + i, val) sorted by p):
//   kap_m <- RN(kap_m a), g <- RN(g a), kg = RN(g k), qg = RN(g q)
//   w_j = csum(B_.j, kg); for each entry of column j: w_j = fma(val, kg_i, w_j);
//         w_j = fma(u_m,j, csum(kap_m, k), w_j) for m < n
//   u = RN(beta RN(v - w)); store (u, k) as delta n
//   o_j: the same with q, over m <= n
//   if n + 1 == W: D = RN(kap_0 u_0^T) then fma over m; M = fma(g, B + entries, D);
//         the K largest |M| (ties: lower p) become the new entries, the rest
//         is requantized as in the per-step mode; g = 1, n = 0.
//
// Thread layout as in the per-step kernel (8 x 8 block per thread, one
// workgroup per state).  Delta keys are decayed and dotted with k and q by
// (delta, 8-row block) pairs.  At the window end the deltas are staged in LDS
// (window <= 16) and D is accumulated in the state block's registers while
// the base codes wait in theirs.
#include "stq_device.h"

namespace stq {
using namespace dev;
namespace {

constexpr int kWMax = 16;     // window length supported by the LDS staging
constexpr int kKMax = 1024;   // compensation entries
constexpr int kCandMax = 1024;  // top-K candidates ranked exactly

// LDS of the window-end, pack and unpack kernels.  The staged deltas are
// dead once D is formed, so the entry and candidate arrays share their space.
template <int DK, int DV>
struct LdsW {
    Lds<DK, DV> b;            // per-step arrays (partials, row/column constants, 1/c', 1/r')
    float gn[DK];             // cumulative gate
    union {
        struct {
            alignas(16) float kst[kWMax][DK];  // decayed delta keys
            alignas(16) float ust[kWMax][DV];  // delta values
        };
        struct {
            uint32_t cix[kKMax];      // compensation index p (old entries; later the candidate list)
            float cvl[kKMax];         // compensation value (during a selection: the histogram,
                                      // then the chosen entries)
            uint32_t ckey[kCandMax];  // candidate keys
            float csv[kCandMax];      // candidate values
        };
    };
    uint32_t cstart[DV + 1];  // old entries of column j: cstart[j] .. cstart[j+1]-1
    int red[2][8];            // block reductions
    uint32_t bc[4];           // broadcasts
};

// LDS of the in-window step; the compensation entries follow in dynamic LDS:
// [K] index, [K] value, and per entry the gated key and query of its row.
template <int DK, int DV>
struct LdsWin {
    Lds<DK, DV> b;
    float kr[DK], qr[DK];     // k and q as fp32
    float ckp[kWMax][DK / 8], cqp[kWMax][DK / 8];  // csum block partials of kap_m . k, kap_m . q
    alignas(16) float ck[kWMax];
    alignas(16) float cq[kWMax];
    uint32_t cstart[DV + 1];  // entries of column j: cstart[j] .. cstart[j+1]-1
};

// Block-wide sum of one int per thread (alternating buffers: one barrier).
template <int NT>
__device__ __forceinline__ int block_sum(int v, int (&red)[2][8], int &phase) {
    constexpr int NW = NT / 64;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    const int t = threadIdx.x;
    if ((t & 63) == 0) red[phase][t >> 6] = v;
    __syncthreads();
    int s = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += red[phase][w];
    phase ^= 1;
    return s;
}

// Block-wide sum of a small non-negative count per thread (< 2^BITS), from
// one wave ballot per bit (alternating buffers: one barrier).
template <int NT, int BITS>
__device__ __forceinline__ int block_count(int v, int (&red)[2][8], int &phase) {
    constexpr int NW = NT / 64;
    int s = 0;
#pragma unroll
    for (int k = 0; k < BITS; ++k) s += (int)__popcll(__ballot((v >> k) & 1)) << k;
    const int t = threadIdx.x;
    if ((t & 63) == 0) red[phase][t >> 6] = s;
    __syncthreads();
    int tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += red[phase][w];
    phase ^= 1;
    return tot;
}

// First index e in [0, n) with a[e] >= x (a sorted ascending).
__device__ __forceinline__ int lower_bound(const uint32_t *a, int n, uint32_t x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] < x) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// Selection works on magnitudes |M| of entries of quantized rows; for finite
// non-negative floats the bit patterns order like the values, which the
// fallback search uses.  Linear index p = j*d_k + i; the thread's entry (r, c)
// has p = pbase + c*d_k + r with pbase = 8*cg*d_k + 8*rg.

// Hides the block's values from the optimizer: magnitudes computed before are
// not carried to later uses (64 more live registers), they are formed again.
__device__ __forceinline__ void opaque_block(float (&x)[8][8]) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) asm volatile("" : "+v"(x[r][c]));
}

// Number of the thread's quantized entries with |M| >= thr.
__device__ __forceinline__ int count_ge(const float (&x)[8][8], const Rows &rw, float thr) {
    int n = 0;
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) n += (rw.w[r] != 16) & (fabsf(x[r][c]) >= thr);
    return n;
}

// Is (|M|, p) of the thread's entry (r, c) among the first K in the order
// (|M| descending, p ascending), given the K-th entry (thr, pk)?
template <int DK>
__device__ __forceinline__ bool chosen(float v, uint32_t p, float thr, uint32_t pk) {
    return (v > thr) || (v == thr && p <= pk);
}

// Radix selection with LDS histograms of 256 bins (8-bit digits).  A pass
// histograms one digit of the keys that match the digits found so far; after
// one barrier every wave scans the bins itself (lane l owns bins 4l .. 4l+3),
// so the digit needs no broadcast.  Three histograms rotate: pass k fills
// hist k % 3 and clears hist (k + 1) % 3, last read in pass k - 2, whose scans
// every wave finished before the barrier of pass k - 1.

// Bits above digit `shift` (the digits already found).
__device__ __forceinline__ uint32_t above_digit(int shift) { return shift >= 24 ? 0u : ~0u << (shift + 8); }

struct Digit {
    uint32_t d;      // the digit
    uint32_t other;  // descending: keys in bins above d; ascending: keys in bins below d
    uint32_t eq;     // keys in bin d
};

// Largest digit d with (keys in bins >= d) >= need (DESC), or smallest digit
// d with (keys in bins <= d) >= need (ascending).  need >= 1 and the
// histogram holds at least need keys.  Called by every lane of a wave.
template <bool DESC>
__device__ __forceinline__ Digit find_digit(const uint32_t *hist, uint32_t need, int lane) {
    const uint4 h = reinterpret_cast<const uint4 *>(hist)[lane];
    const uint32_t local = h.x + h.y + h.z + h.w;
    uint32_t S = local;  // keys in the bins of lanes >= lane (DESC) or <= lane
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = DESC ? __shfl_down(S, off, 64) : __shfl_up(S, off, 64);
        if (DESC ? lane + off < 64 : lane >= off) S += o;
    }
    int d = -1;
    uint32_t other = 0, eq = 0;
    if (DESC) {
        const uint32_t s3 = S - local + h.w, s2 = s3 + h.z, s1 = s2 + h.y, s0 = s1 + h.x;
        if (s3 >= need) { d = 4 * lane + 3; other = s3 - h.w; eq = h.w; }
        else if (s2 >= need) { d = 4 * lane + 2; other = s2 - h.z; eq = h.z; }
        else if (s1 >= need) { d = 4 * lane + 1; other = s1 - h.y; eq = h.y; }
        else if (s0 >= need) { d = 4 * lane; other = s0 - h.x; eq = h.x; }
    } else {
        const uint32_t p0 = S - local + h.x, p1 = p0 + h.y, p2 = p1 + h.z, p3 = p2 + h.w;
        if (p0 >= need) { d = 4 * lane; other = p0 - h.x; eq = h.x; }
        else if (p1 >= need) { d = 4 * lane + 1; other = p1 - h.y; eq = h.y; }
        else if (p2 >= need) { d = 4 * lane + 2; other = p2 - h.z; eq = h.z; }
        else if (p3 >= need) { d = 4 * lane + 3; other = p3 - h.w; eq = h.w; }
    }
    // the counts are monotone over the lanes, so the lanes holding a digit
    // are 0 .. L (DESC: the answer is lane L) or L .. 63 (the answer is L)
    const unsigned long long m = __ballot(d >= 0);
    const int L = DESC ? 63 - __clzll((long long)m) : __ffsll((long long)m) - 1;
    return Digit{(uint32_t)__shfl(d, L, 64), (uint32_t)__shfl((int)other, L, 64),
                 (uint32_t)__shfl((int)eq, L, 64)};
}

template <int NT>
__device__ __forceinline__ void hist_clear(uint32_t *hist, int t) {
    for (int i = t; i < 256; i += NT) hist[i] = 0u;
}

// Select the K entries of largest |M| (ties: lower p) among the quantized rows
// of the state held in x; write them sorted by p to the head's compensation
// arrays and set them to 0 in x (so they are left out of both scale maxima
// and get code 0).
template <int DK, int DV>
__device__ void select_comps(const Args &A, const HeadDesc &hd, uint8_t *R, const Rows &rw,
                             float (&x)[8][8], LdsW<DK, DV> &sm, int t, int rg, int cg) {
    constexpr int NT = DK * DV / 64;
    const int K = A.comps;
    if (K <= 0) return;
    const uint32_t pbase = (uint32_t)(8 * cg * DK + 8 * rg);
    int phase = 0;
    float thr = 0.0f;        // the K-th entry is (thr, pk)
    uint32_t pk = 0;
    bool exact = false;
    int total = 0;  // candidates in LDS (when exact)

    // 1) the K-th largest of the per-thread maxima bounds the K-th |M| from
    //    below; two radix passes find its top 16 bits, t0 (its low bits
    //    cleared: still a bound), and the largest maximum comes with them
    float tmax = -1.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c)
            if (rw.w[r] != 16) tmax = fmaxf(tmax, fabsf(x[r][c]));
    if (K <= NT) {
        // three histograms in the entry-value array (unused until the chosen
        // entries are gathered); the keys of magnitudes order like the values,
        // and a thread without quantized entries has key 0
        uint32_t *hists = reinterpret_cast<uint32_t *>(sm.cvl);
        int pass = 0;
        const int lane = t & 63;
        const uint32_t key = tmax >= 0.0f ? __float_as_uint(tmax) : 0u;
        uint32_t lo = 0, need = K;
        hist_clear<NT>(hists, t);
        if (t == 0) sm.bc[3] = 0u;
        __syncthreads();
        atomicMax(&sm.bc[3], key);
        for (int shift = 24; shift >= 16; shift -= 8, ++pass) {
            uint32_t *hist = hists + 256 * (pass % 3);
            hist_clear<NT>(hists + 256 * ((pass + 1) % 3), t);
            if (((key ^ lo) & above_digit(shift)) == 0u) atomicAdd(&hist[(key >> shift) & 255u], 1u);
            __syncthreads();
            const Digit g = find_digit<true>(hist, need, lane);
            lo |= g.d << shift;
            need -= g.other;
        }
        const float t0 = __uint_as_float(lo);
        const uint32_t kmax = sm.bc[3];
        // 2) compact the candidates |M| >= t0 into LDS when they are few
        const int mine = count_ge(x, rw, t0);
        opaque_block(x);
        total = block_sum<NT>(mine, sm.red, phase);
        if (total <= kCandMax) {
            if (t == 0) sm.bc[1] = 0;
            __syncthreads();
            int base = mine ? (int)atomicAdd(&sm.bc[1], (uint32_t)mine) : 0;
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const float v = fabsf(x[r][c]);
                    if (rw.w[r] != 16 && v >= t0) {
                        sm.ckey[base] = __float_as_uint(v);
                        sm.cix[base] = pbase + (uint32_t)(c * DK + r);
                        sm.csv[base] = x[r][c];
                        ++base;
                    }
                }
            opaque_block(x);
            __syncthreads();
            // 3) the K-th candidate in the order (|M| descending, p ascending):
            //    radix passes over the |M| bits below the highest one where t0
            //    and the largest candidate differ (the bits above are common to
            //    every candidate), then, if some of its ties are left out,
            //    over the p of those ties
            const int top = (lo ^ kmax) ? 31 - __builtin_clz(lo ^ kmax) : -1;
            uint32_t P = top >= 0 ? lo & ~((2u << top) - 1u) : lo;
            uint32_t ties = (uint32_t)total;  // candidates equal to P (all of them if top < 0)
            need = K;
            for (int shift = top >= 0 ? (top >> 3) << 3 : -8; shift >= 0; shift -= 8, ++pass) {
                uint32_t *hist = hists + 256 * (pass % 3);
                hist_clear<NT>(hists + 256 * ((pass + 1) % 3), t);
                const uint32_t hm = above_digit(shift);
#pragma unroll
                for (int k = 0; k < kCandMax / NT; ++k) {
                    const int e = t + k * NT;
                    if (e >= total) break;
                    const uint32_t v = sm.ckey[e];
                    if (((v ^ P) & hm) == 0u) atomicAdd(&hist[(v >> shift) & 255u], 1u);
                }
                __syncthreads();
                const Digit g = find_digit<true>(hist, need, lane);
                P |= g.d << shift;
                need -= g.other;
                ties = g.eq;
            }
            uint32_t X = 0xffffffffu;  // every tie chosen
            if (need < ties) {
                X = 0;
                for (int shift = 8; shift >= 0; shift -= 8, ++pass) {
                    uint32_t *hist = hists + 256 * (pass % 3);
                    hist_clear<NT>(hists + 256 * ((pass + 1) % 3), t);
                    const uint32_t hm = above_digit(shift);
#pragma unroll
                    for (int k = 0; k < kCandMax / NT; ++k) {
                        const int e = t + k * NT;
                        if (e >= total) break;
                        const uint32_t q = sm.cix[e];
                        if (sm.ckey[e] == P && ((q ^ X) & hm) == 0u) atomicAdd(&hist[(q >> shift) & 255u], 1u);
                    }
                    __syncthreads();
                    const Digit g = find_digit<false>(hist, need, lane);
                    X |= g.d << shift;
                    need -= g.other;
                }
            }
            // the histograms are read until here: the gather below reuses them
            __syncthreads();
            thr = __uint_as_float(P);
            pk = X;
            exact = true;
        }
    }
    if (!exact) {
        // fallback: bit-serial search of the K-th |M| over the whole state,
        // then of the tie position
        // (opaque_block in the loops: per-entry values hoisted out of them
        // would hold a register each for the whole loop)
        uint32_t P = 0;
        for (int bit = 30; bit >= 0; --bit) {
            opaque_block(x);
            const uint32_t cand = P | (1u << bit);
            if (block_sum<NT>(count_ge(x, rw, __uint_as_float(cand)), sm.red, phase) >= K) P = cand;
        }
        thr = __uint_as_float(P);
        int above = 0;
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int c = 0; c < 8; ++c) above += (rw.w[r] != 16) & (fabsf(x[r][c]) > thr);
        const int need = K - block_sum<NT>(above, sm.red, phase);
        uint32_t X = 0;
        for (int bit = 15; bit >= 0; --bit) {
            opaque_block(x);
            const uint32_t cand = X | (1u << bit);
            int m2 = 0;
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    m2 += (rw.w[r] != 16) & (fabsf(x[r][c]) == thr) & (pbase + (uint32_t)(c * DK + r) < cand);
            if (block_sum<NT>(m2, sm.red, phase) < need) X = cand;
        }
        pk = X;
    }

    // the chosen entries (index p in sp, value in sv), then ranked by p for
    // storage; each is marked in a 64-bit mask per owner thread (bit 8 r + c
    // of its block, kept in the column-partial array, unused until the
    // requantization) and then set to 0 in x
    uint32_t *sp = sm.cix;
    float *sv = sm.cvl;
    uint32_t *zm = reinterpret_cast<uint32_t *>(&sm.b.colp[0][0]);
    if (t == 0) sm.bc[1] = 0;
    if (exact) {
        // they are among the candidates in LDS: gathered from there (K <= NT
        // here, so they fit in the histogram's array)
        sp = reinterpret_cast<uint32_t *>(sm.cvl);
        sv = sm.cvl + kKMax / 2;
        zm[2 * t] = 0u;
        zm[2 * t + 1] = 0u;
        __syncthreads();
        constexpr int CG = DV / 8;
#pragma unroll
        for (int k = 0; k < kCandMax / NT; ++k) {
            const int e = t + k * NT;
            if (e >= total) break;
            const uint32_t v = sm.ckey[e], p = sm.cix[e];
            if (chosen<DK>(__uint_as_float(v), p, thr, pk)) {
                const uint32_t slot = atomicAdd(&sm.bc[1], 1u);
                sp[slot] = p;
                sv[slot] = sm.csv[e];
                const uint32_t j = p / DK, i = p - j * DK;
                const uint32_t owner = (i >> 3) * CG + (j >> 3), bit = (i & 7u) * 8u + (j & 7u);
                atomicOr(&zm[2 * owner + (bit >> 5)], 1u << (bit & 31u));
            }
        }
    } else {
        __syncthreads();
        int mine = 0;
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int c = 0; c < 8; ++c)
                mine += (rw.w[r] != 16) & chosen<DK>(fabsf(x[r][c]), pbase + (uint32_t)(c * DK + r), thr, pk);
        int base = mine ? (int)atomicAdd(&sm.bc[1], (uint32_t)mine) : 0;
        uint32_t zlo = 0u, zhi = 0u;
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const uint32_t p = pbase + (uint32_t)(c * DK + r);
                if (rw.w[r] != 16 && chosen<DK>(fabsf(x[r][c]), p, thr, pk)) {
                    sm.cix[base] = p;
                    sm.cvl[base] = x[r][c];
                    ++base;
                    const int bit = r * 8 + c;
                    if (bit < 32) zlo |= 1u << bit; else zhi |= 1u << (bit - 32);
                }
            }
        zm[2 * t] = zlo;
        zm[2 * t + 1] = zhi;
    }
    __syncthreads();
    {
        const uint32_t zlo = zm[2 * t], zhi = zm[2 * t + 1];
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int bit = r * 8 + c;
                if (((bit < 32 ? zlo >> bit : zhi >> (bit - 32)) & 1u) != 0u) x[r][c] = 0.0f;
            }
    }
    __syncthreads();
    for (int e = t; e < K; e += NT) {
        const uint32_t p = sp[e];
        // rank = entries of smaller index, four per LDS read (sp is 16-byte aligned)
        int rank = 0;
        const uint4 *s4 = reinterpret_cast<const uint4 *>(sp);
#pragma unroll 4
        for (int f = 0; f < (K >> 2); ++f) {
            const uint4 q = s4[f];
            rank += (int)(q.x < p) + (int)(q.y < p) + (int)(q.z < p) + (int)(q.w < p);
        }
        for (int f = K & ~3; f < K; ++f) rank += sp[f] < p;
        reinterpret_cast<uint16_t *>(R + hd.cidx)[rank] = (uint16_t)p;
        reinterpret_cast<float *>(R + hd.cval)[rank] = sv[e];
    }
    __syncthreads();
}

// Base B of one row piece: RN(RN(n r) c) for a quantized row (n r is exact),
// the stored fp16 values for a pivot row.  No compensation entries.
template <int DK, int DV>
__device__ __forceinline__ void base_row(int w, uint4 raw, const Lds<DK, DV> &sm, int i,
                                         const float (&cc)[8], float (&x)[8]) {
    if (w == 16) {
        const uint32_t hv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            x[2 * c] = f16v(hv[c]);
            x[2 * c + 1] = f16v(hv[c] >> 16);
        }
    } else {
        dequant_row(raw, w, sm.g[i], sm.g16[i], sm.nog[i], x);
#pragma unroll
        for (int c = 0; c < 8; ++c) x[c] = x[c] * cc[c];
    }
}

template <int DK, int DV>
__device__ __forceinline__ void base_block(const Rows &rw, const uint4 (&raw)[8], const Lds<DK, DV> &sm,
                                           int rg, const float (&cc)[8], float (&x)[8][8]) {
#pragma unroll
    for (int r = 0; r < 8; ++r) base_row<DK, DV>(rw.w[r], raw[r], sm, 8 * rg + r, cc, x[r]);
}

// Row and column constants of the base dequantization (row scale r: in g,
// r/16 in g16, -2^(w-1) r in nog; column scales in cf).
template <int DK, int DV, int W>
__device__ __forceinline__ void base_constants(const Args &A, const HeadDesc &hd, uint32_t rraw, uint32_t craw,
                                               Lds<DK, DV> &sm, int t) {
    const bool quant = has_quant<W>(hd);
    if (t < DK) {
        const int w = width_of<W>(A, hd, t);
        const float rl = dec_scale(rraw, A.rs16, t & 1);
        const float ri = (quant && w != 16) ? rl : 0.0f;
        sm.g[t] = ri;
        sm.g16[t] = ri * 0.0625f;
        sm.nog[t] = w != 16 ? -(float)(1 << (w - 1)) * ri : 0.0f;
    }
    if (t < DV) {
        const float c = dec_scale(craw, 1, t & 1);
        sm.cf[t] = (quant && A.cs16) ? c : 1.0f;
    }
}

// The same from the head's stored scales (a head without scales has offset 0
// here: still inside its region).
template <int DK, int DV, int W>
__device__ __forceinline__ void base_constants(const Args &A, const HeadDesc &hd, const uint8_t *R,
                                               Lds<DK, DV> &sm, int t) {
    const uint32_t rraw = ld_dword(R + hd.rs, A.rs16, t < DK ? t : 0);
    const uint32_t craw = ld_dword(R + hd.cs, 1, t < DV ? t : 0);
    base_constants<DK, DV, W>(A, hd, rraw, craw, sm, t);
}

template <int DK, int DV, int W>
__device__ __forceinline__ void win_tile(const Args &A, const HeadDesc &hd, uint8_t *R, size_t unit,
                                         LdsWin<DK, DV> &sm, uint32_t *cix, float *cvl, float *kge, float *qge,
                                         int t, int rg, int cg) {
    constexpr int NT = DK * DV / 64, RG = DK / 8;
    const int W_ = A.window;
    const int K = A.comps;
    // The loads below do not depend on the delta count, so they are all
    // issued before it arrives (no load waits for another).
    Rows rw;
    row_geometry<DV, W>(A, hd, rg, rw);
    uint4 raw[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) raw[r] = load_piece(R + rw.ro[r], cg, rw.w[r]);
    float *gmem = reinterpret_cast<float *>(R + hd.g);
    float *du = reinterpret_cast<float *>(R + hd.du);
    float *dkap = reinterpret_cast<float *>(R + hd.dkap);

    // per key row / value column inputs and constants
    Inputs in;
    fetch_inputs<DK, DV>(A, hd, R, unit, t, in);
    const float gold = gmem[t < DK ? t : 0];
    // this thread's first compensation entry (more below if K > NT)
    const uint16_t *cidx = reinterpret_cast<const uint16_t *>(R + hd.cidx);
    const float *cval = reinterpret_cast<const float *>(R + hd.cval);
    uint32_t ci0 = 0;
    float cv0 = 0.0f;
    if (t < K) {
        ci0 = cidx[t];
        cv0 = cval[t];
    }
    const int n = *reinterpret_cast<const int32_t *>(R + hd.wn);
    base_constants<DK, DV, W>(A, hd, in.r, in.c, sm.b, t);
    const float beta = in.beta;
    float vv = 0.0f, gnew = 0.0f;
    if (t < DK) {
        const float a = in.a;
        const float k = dec_io(in.k, A.io_bf16, t & 1);
        const float q = dec_io(in.q, A.io_bf16, t & 1);
        const float g = gold * a;
        sm.b.af[t] = a;
        sm.kr[t] = k;
        sm.qr[t] = q;
        sm.b.kf[t] = g * k;
        sm.b.qf[t] = g * q;
        gnew = g;
    }
    if (t < DV) vv = dec_io(in.v, A.io_bf16, t & 1);
    if (t < K) {
        cix[t] = ci0;
        cvl[t] = cv0;
    }
    keep_inputs(in);
    asm volatile("" ::"v"(gold), "v"(ci0), "v"(cv0));  // (as keep_inputs)
    for (int e = t + NT; e < K; e += NT) {
        cix[e] = cidx[e];
        cvl[e] = cval[e];
    }
    if (n < 0 || n >= W_) {
        // a delta count outside [0, W) is not a state this library wrote:
        // nothing is stored into it
        if (t < DV) A.o[unit * DV + t] = __builtin_nanf("");
        return;
    }
    if (t < DK) gmem[t] = gnew;
    // the first (delta, 8-row block) of delta keys that this thread decays,
    // in flight across the barrier (the delta count is known by now)
    float kap0[8];
    {
        const int m0 = t / RG, i0 = 8 * (t - m0 * RG);
        if (m0 < n) {
            const float4 *p = reinterpret_cast<const float4 *>(dkap + (size_t)m0 * DK + i0);
            const float4 a0 = p[0], a1 = p[1];
            kap0[0] = a0.x; kap0[1] = a0.y; kap0[2] = a0.z; kap0[3] = a0.w;
            kap0[4] = a1.x; kap0[5] = a1.y; kap0[6] = a1.z; kap0[7] = a1.w;
        }
    }
    __syncthreads();

    // column ranges of the entries (sorted by p = j*d_k + i), and each
    // entry's gated key and query (the operands of its fma in w and o)
    if (K == 0) {
        for (int j = t; j <= DV; j += NT) sm.cstart[j] = 0;
    }
    for (int e = t; e < K; e += NT) {
        const uint32_t p = cix[e];
        const int j = (int)(p / DK), i = (int)(p - (uint32_t)j * DK);
        kge[e] = sm.b.kf[i];
        qge[e] = sm.b.qf[i];
        const int jp = e > 0 ? (int)(cix[e - 1] / DK) : -1;
        for (int jj = jp + 1; jj <= j; ++jj) sm.cstart[jj] = e;
        if (e == K - 1)
            for (int jj = j + 1; jj <= DV; ++jj) sm.cstart[jj] = K;
    }

    // delta keys: decay, store back, block partials of kap . k and kap . q
    for (int pr = t; pr < (n + 1) * RG; pr += NT) {
        const int m = pr / RG, blk = pr - m * RG, i0 = 8 * blk;
        float kap[8];
        if (m < n) {
            float4 *p = reinterpret_cast<float4 *>(dkap + (size_t)m * DK + i0);
            if (pr == t) {
#pragma unroll
                for (int r = 0; r < 8; ++r) kap[r] = kap0[r];
            } else {
                const float4 a0 = p[0], a1 = p[1];
                kap[0] = a0.x; kap[1] = a0.y; kap[2] = a0.z; kap[3] = a0.w;
                kap[4] = a1.x; kap[5] = a1.y; kap[6] = a1.z; kap[7] = a1.w;
            }
#pragma unroll
            for (int r = 0; r < 8; ++r) kap[r] = kap[r] * sm.b.af[i0 + r];
            p[0] = make_float4(kap[0], kap[1], kap[2], kap[3]);
            p[1] = make_float4(kap[4], kap[5], kap[6], kap[7]);
            float s = kap[0] * sm.kr[i0];
#pragma unroll
            for (int r = 1; r < 8; ++r) s = fma_(kap[r], sm.kr[i0 + r], s);
            sm.ckp[m][blk] = s;
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r) kap[r] = sm.kr[i0 + r];
        }
        float s = kap[0] * sm.qr[i0];
#pragma unroll
        for (int r = 1; r < 8; ++r) s = fma_(kap[r], sm.qr[i0 + r], s);
        sm.cqp[m][blk] = s;
    }

    // base read / output partials
    float cc[8], kk[8], qq[8];
    lds_read8(&sm.b.cf[8 * cg], cc, 0);
    lds_read8(&sm.b.kf[8 * rg], kk, 0);
    lds_read8(&sm.b.qf[8 * rg], qq, 0);
    float x[8][8];
    base_block<DK, DV>(rw, raw, sm.b, rg, cc, x);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        float s = x[0][c] * kk[0], s2 = x[0][c] * qq[0];
#pragma unroll
        for (int r = 1; r < 8; ++r) {
            s = fma_(x[r][c], kk[r], s);
            s2 = fma_(x[r][c], qq[r], s2);
        }
        sm.b.colp[c][t] = s;
        sm.b.colm[c][t] = s2;
    }
    __syncthreads();
    // the stored delta values of column t (read only by thread t), loaded
    // once the state block is dead so that they do not add to its registers
    float um[kWMax];
    if (t < DV) {
#pragma unroll
        for (int m = 0; m < kWMax; ++m) um[m] = m < n ? du[(size_t)m * DV + t] : 0.0f;
    }
    float w0 = 0.0f, o0 = 0.0f;
    if (t < DV) {
        w0 = col_sum<DK, DV>(sm.b, t);
        const float *p = &sm.b.colm[t & 7][t >> 3];
        o0 = p[0];
#pragma unroll
        for (int g = 1; g < RG; ++g) o0 = o0 + p[g * (DV / 8)];
    }
    if (t <= n) {
        float s = 0.0f, s2 = sm.cqp[t][0];
        if (t < n) s = sm.ckp[t][0];
#pragma unroll
        for (int g = 1; g < RG; ++g) {
            if (t < n) s = s + sm.ckp[t][g];
            s2 = s2 + sm.cqp[t][g];
        }
        sm.ck[t] = s;
        sm.cq[t] = s2;
    }
    __syncthreads();

    if (t < DV) {
        // w and o of column j: the entries of the column in index order, then
        // the stored deltas; the two chains are independent and interleaved
        const int j = t;
        const int lo = (int)sm.cstart[j], hi = (int)sm.cstart[j + 1];
        float ck[kWMax], cq[kWMax];
#pragma unroll
        for (int m = 0; m < kWMax; m += 4) {
            const float4 a = *reinterpret_cast<const float4 *>(&sm.ck[m]);
            const float4 c = *reinterpret_cast<const float4 *>(&sm.cq[m]);
            ck[m] = a.x; ck[m + 1] = a.y; ck[m + 2] = a.z; ck[m + 3] = a.w;
            cq[m] = c.x; cq[m + 1] = c.y; cq[m + 2] = c.z; cq[m + 3] = c.w;
        }
        const float cqn = sm.cq[n];
        float w = w0, o = o0;
#pragma unroll 4
        for (int e = lo; e < hi; ++e) {
            const float v = cvl[e];
            w = fma_(v, kge[e], w);
            o = fma_(v, qge[e], o);
        }
#pragma unroll
        for (int m = 0; m < kWMax; ++m) {
            if (m < n) {
                w = fma_(um[m], ck[m], w);
                o = fma_(um[m], cq[m], o);
            }
        }
        const float u = beta * (vv - w);
        du[(size_t)n * DV + j] = u;
        o = fma_(u, cqn, o);
        A.o[unit * DV + j] = o;
    }
    if (t < DK) dkap[(size_t)n * DK + t] = sm.kr[t];
    // at the W-th delta the count reaches W; the window-end kernel closes it,
    // told by the pool's flag holding this call's token
    if (t == 0) {
        *reinterpret_cast<int32_t *>(R + hd.wn) = n + 1;
        if (n + 1 == A.window) *A.end_flag = A.token;
    }
}

// Window end of one state holding W deltas: M = fma(g, B + entries, D) with
// D = RN(kap_0 u_0^T) then fma over the deltas; the K largest |M| become the
// new compensation entries, the rest is requantized; g = 1, n = 0.
template <int DK, int DV, int W>
__device__ __forceinline__ void end_tile(const Args &A, const HeadDesc &hd, uint8_t *R, size_t unit,
                                         LdsW<DK, DV> &sm, int t, int rg, int cg) {
    constexpr int NT = DK * DV / 64;
    const int n = A.window;
    const int K = A.comps;
    Rows rw;
    row_geometry<DV, W>(A, hd, rg, rw);
    uint4 raw[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) raw[r] = load_piece(R + rw.ro[r], cg, rw.w[r]);
    float *gmem = reinterpret_cast<float *>(R + hd.g);
    const float *du = reinterpret_cast<const float *>(R + hd.du);
    const float *dkap = reinterpret_cast<const float *>(R + hd.dkap);
    base_constants<DK, DV, W>(A, hd, R, sm.b, t);
    {
        // stage the W deltas in LDS: every 16-byte load is issued before the
        // first LDS write, so the staging costs one memory round trip
        constexpr int PER = (kWMax * (DK > DV ? DK : DV) / 4 + NT - 1) / NT;
        const int nk = n * DK / 4, nu = n * DV / 4;
        const float4 *ks = reinterpret_cast<const float4 *>(dkap);
        const float4 *us = reinterpret_cast<const float4 *>(du);
        float4 kv[PER], uv[PER];
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int e = t + p * NT;
            kv[p] = ks[e < nk ? e : 0];  // index 0 is always valid (n >= 1)
            uv[p] = us[e < nu ? e : 0];
        }
        float4 *kd = reinterpret_cast<float4 *>(&sm.kst[0][0]);
        float4 *ud = reinterpret_cast<float4 *>(&sm.ust[0][0]);
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int e = t + p * NT;
            if (e < nk) kd[e] = kv[p];
            if (e < nu) ud[e] = uv[p];
        }
    }
    if (t < DK) sm.gn[t] = gmem[t];
    // the old entries go to LDS once the staged deltas are used up (they share
    // the space); thread t holds entry t, and the index before it, meanwhile
    const uint16_t *cidx = reinterpret_cast<const uint16_t *>(R + hd.cidx);
    const float *cval = reinterpret_cast<const float *>(R + hd.cval);
    uint32_t pe = 0, pp = 0;
    float ve = 0.0f;
    if (t < K) {
        pe = cidx[t];
        ve = cval[t];
        pp = t > 0 ? cidx[t - 1] : 0u;
    }
    __syncthreads();
    float x[8][8];
    {
        float kq[8], uq[8];
        lds_read8(&sm.kst[0][8 * rg], kq, 0);
        lds_read8(&sm.ust[0][8 * cg], uq, 0);
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int c = 0; c < 8; ++c) x[r][c] = kq[r] * uq[c];
        for (int m = 1; m < n; ++m) {
            lds_read8(&sm.kst[m][8 * rg], kq, 0);
            lds_read8(&sm.ust[m][8 * cg], uq, 0);
#pragma unroll
            for (int r = 0; r < 8; ++r)
#pragma unroll
                for (int c = 0; c < 8; ++c) x[r][c] = fma_(kq[r], uq[c], x[r][c]);
        }
    }
    __syncthreads();  // the staged deltas are no longer read
    // old entries into LDS, and the range of each column's entries (sorted by
    // p = j*d_k + i)
    if (K == 0) {
        for (int j = t; j <= DV; j += NT) sm.cstart[j] = 0;
    }
    for (int e = t; e < K; e += NT) {
        const uint32_t p = e == t ? pe : cidx[e];
        const uint32_t q = e == t ? pp : cidx[e - 1];
        sm.cix[e] = p;
        sm.cvl[e] = e == t ? ve : cval[e];
        const int j = (int)(p / DK);
        const int jp = e > 0 ? (int)(q / DK) : -1;
        for (int jj = jp + 1; jj <= j; ++jj) sm.cstart[jj] = e;
        if (e == K - 1)
            for (int jj = j + 1; jj <= DV; ++jj) sm.cstart[jj] = K;
    }
    __syncthreads();
    float gg[8], cc[8];
    lds_read8(&sm.gn[8 * rg], gg, 0);
    lds_read8(&sm.b.cf[8 * cg], cc, 0);
    // M = fma(g, B, D): compensation entries at their positions first
    uint64_t done = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t p0 = (uint32_t)((8 * cg + c) * DK + 8 * rg);
        const int c0 = (int)sm.cstart[8 * cg + c], c1 = (int)sm.cstart[8 * cg + c + 1];
        const int lo = c0 + lower_bound(sm.cix + c0, c1 - c0, p0);
        for (int e = lo; e < c1 && sm.cix[e] < p0 + 8; ++e) {
            const int rr = (int)(sm.cix[e] - p0);
            const float val = sm.cvl[e];
#pragma unroll
            for (int r = 0; r < 8; ++r)
                if (r == rr) x[r][c] = fma_(gg[r], val, x[r][c]);
            done |= 1ull << (rr * 8 + c);
        }
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        float B[8];
        base_row<DK, DV>(rw.w[r], raw[r], sm.b, 8 * rg + r, cc, B);
        const uint32_t dr = (uint32_t)(done >> (8 * r)) & 0xffu;
#pragma unroll
        for (int c = 0; c < 8; ++c)
            if (!((dr >> c) & 1u)) x[r][c] = fma_(gg[r], B[c], x[r][c]);
    }
    __syncthreads();  // old entries are no longer read from LDS
    select_comps<DK, DV>(A, hd, R, rw, x, sm, t, rg, cg);
    requant_store<DK, DV, W, false>(A, hd, R, rw, x, sm.b, t, rg, cg, false, unit);
    if (t < DK) gmem[t] = 1.0f;
    if (t == 0) *reinterpret_cast<int32_t *>(R + hd.wn) = 0;
}

// Four waves per SIMD (128 VGPRs) for the uniform-width instantiations: the
// few spills cost less than the lost occupancy (the window end is ~20 %
// faster at d = 128); the per-row path would spill too much and keeps three.
template <int DK, int DV, bool MIXED>
__global__ void __launch_bounds__(DK * DV / 64) __attribute__((amdgpu_waves_per_eu(MIXED ? 3 : 4)))
k_win_end(Args A) {
    constexpr int CG = DV / 8;
    __shared__ LdsW<DK, DV> sm;
    // no state of this call filled its window (the flag holds an earlier
    // token): one load, and every workgroup is done
    if (*A.end_flag != A.token) return;
    const size_t unit = blockIdx.x;
    const int b = (int)(unit / (size_t)A.H);
    const int h = (int)(unit - (size_t)b * A.H);
    const int t = threadIdx.x, rg = t / CG, cg = t - rg * CG;
    const int slot = A.slot_ids[b];
    if (slot < 0 || slot >= A.nslots) return;
    const HeadDesc hd = A.heads[h];  // copied before any store, as in k_win
    uint8_t *R = A.slots + (size_t)slot * A.slot_bytes + hd.off;
    if (*reinterpret_cast<const int32_t *>(R + hd.wn) != A.window) return;
    switch (head_width(hd)) {
        case 4: end_tile<DK, DV, 4>(A, hd, R, unit, sm, t, rg, cg); break;
        case 6: end_tile<DK, DV, 6>(A, hd, R, unit, sm, t, rg, cg); break;
        case 8: end_tile<DK, DV, 8>(A, hd, R, unit, sm, t, rg, cg); break;
        case 16: end_tile<DK, DV, 16>(A, hd, R, unit, sm, t, rg, cg); break;
        default:
            if (MIXED) end_tile<DK, DV, 0>(A, hd, R, unit, sm, t, rg, cg);
            break;
    }
}

template <int DK, int DV, bool MIXED>
__global__ void __launch_bounds__(DK * DV / 64) k_win(Args A) {
    constexpr int CG = DV / 8;
    __shared__ LdsWin<DK, DV> sm;
    extern __shared__ uint32_t win_entries[];  // [K] index, value, gated key, gated query
    uint32_t *cix = win_entries;
    float *cvl = reinterpret_cast<float *>(win_entries + A.comps);
    float *kge = cvl + A.comps;
    float *qge = kge + A.comps;
    const size_t unit = blockIdx.x;
    const int b = (int)(unit / (size_t)A.H);
    const int h = (int)(unit - (size_t)b * A.H);
    const int t = threadIdx.x, rg = t / CG, cg = t - rg * CG;
    const int slot = A.slot_ids[b];
    // the descriptor copied before any store (fields read after a store into
    // the pool would be reloaded by vector loads)
    const HeadDesc hd = A.heads[h];
    if (slot < 0 || slot >= A.nslots) {
        if (t < DV) A.o[unit * DV + t] = __builtin_nanf("");
        return;
    }
    uint8_t *R = A.slots + (size_t)slot * A.slot_bytes + hd.off;
    switch (head_width(hd)) {
        case 4: win_tile<DK, DV, 4>(A, hd, R, unit, sm, cix, cvl, kge, qge, t, rg, cg); break;
        case 6: win_tile<DK, DV, 6>(A, hd, R, unit, sm, cix, cvl, kge, qge, t, rg, cg); break;
        case 8: win_tile<DK, DV, 8>(A, hd, R, unit, sm, cix, cvl, kge, qge, t, rg, cg); break;
        case 16: win_tile<DK, DV, 16>(A, hd, R, unit, sm, cix, cvl, kge, qge, t, rg, cg); break;
        default:
            if (MIXED) win_tile<DK, DV, 0>(A, hd, R, unit, sm, cix, cvl, kge, qge, t, rg, cg);
            break;
    }
}

// stq_pack for the windowed layout: compensation entries chosen from the fp32
// state, the rest requantized, g = 1, no deltas (delta storage cleared).
template <int DK, int DV, int W>
__device__ __forceinline__ void pack_win_tile(const Args &A, const HeadDesc &hd, uint8_t *R, size_t unit,
                                              LdsW<DK, DV> &sm, int t, int rg, int cg) {
    constexpr int NT = DK * DV / 64;
    Rows rw;
    row_geometry<DV, W>(A, hd, rg, rw);
    float x[8][8];
    const float *src = A.state + unit * DK * DV;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const float4 *p = reinterpret_cast<const float4 *>(src + (size_t)(8 * rg + r) * DV + 8 * cg);
        const float4 a = p[0], b = p[1];
        x[r][0] = a.x; x[r][1] = a.y; x[r][2] = a.z; x[r][3] = a.w;
        x[r][4] = b.x; x[r][5] = b.y; x[r][6] = b.z; x[r][7] = b.w;
    }
    select_comps<DK, DV>(A, hd, R, rw, x, sm, t, rg, cg);
    requant_store<DK, DV, W, false>(A, hd, R, rw, x, sm.b, t, rg, cg, false, unit);
    float *g = reinterpret_cast<float *>(R + hd.g);
    float *du = reinterpret_cast<float *>(R + hd.du);
    float *dkap = reinterpret_cast<float *>(R + hd.dkap);
    for (int i = t; i < DK; i += NT) g[i] = 1.0f;
    for (int e = t; e < A.window * DV; e += NT) du[e] = 0.0f;
    for (int e = t; e < A.window * DK; e += NT) dkap[e] = 0.0f;
    if (t == 0) *reinterpret_cast<int32_t *>(R + hd.wn) = 0;
}

template <int DK, int DV, bool MIXED>
__global__ void __launch_bounds__(DK * DV / 64) k_pack_win(Args A) {
    constexpr int CG = DV / 8;
    __shared__ LdsW<DK, DV> sm;
    const size_t unit = blockIdx.x;
    const int b = (int)(unit / (size_t)A.H);
    const int h = (int)(unit - (size_t)b * A.H);
    const int t = threadIdx.x, rg = t / CG, cg = t - rg * CG;
    const int slot = A.slot_ids[b];
    if (slot < 0 || slot >= A.nslots) return;
    const HeadDesc &hd = A.heads[h];
    uint8_t *R = A.slots + (size_t)slot * A.slot_bytes + hd.off;
    switch (head_width(hd)) {
        case 4: pack_win_tile<DK, DV, 4>(A, hd, R, unit, sm, t, rg, cg); break;
        case 6: pack_win_tile<DK, DV, 6>(A, hd, R, unit, sm, t, rg, cg); break;
        case 8: pack_win_tile<DK, DV, 8>(A, hd, R, unit, sm, t, rg, cg); break;
        case 16: pack_win_tile<DK, DV, 16>(A, hd, R, unit, sm, t, rg, cg); break;
        default:
            if (MIXED) pack_win_tile<DK, DV, 0>(A, hd, R, unit, sm, t, rg, cg);
            break;
    }
}

// stq_unpack for the windowed layout: M = fma(g, B + entries, D) with D the
// stored deltas (or B alone when there are none).
template <int DK, int DV>
__global__ void __launch_bounds__(DK * DV / 64) k_unpack_win(Args A) {
    constexpr int CG = DV / 8;
    __shared__ LdsW<DK, DV> sm;
    const size_t unit = blockIdx.x;
    const int b = (int)(unit / (size_t)A.H);
    const int h = (int)(unit - (size_t)b * A.H);
    const int t = threadIdx.x, rg = t / CG, cg = t - rg * CG;
    const int slot = A.slot_ids[b];
    float *dst = A.state + unit * DK * DV;
    if (slot < 0 || slot >= A.nslots) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int c = 0; c < 8; ++c) dst[(size_t)(8 * rg + r) * DV + 8 * cg + c] = __builtin_nanf("");
        return;
    }
    const HeadDesc &hd = A.heads[h];
    const uint8_t *R = A.slots + (size_t)slot * A.slot_bytes + hd.off;
    int n = *reinterpret_cast<const int32_t *>(R + hd.wn);
    if (n < 0 || n >= A.window) n = 0;
    const int K = A.comps;
    Rows rw;
    row_geometry<DV, 0>(A, hd, rg, rw);
    uint4 raw[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) raw[r] = load_piece(R + rw.ro[r], cg, rw.w[r]);
    base_constants<DK, DV, 0>(A, hd, R, sm.b, t);
    for (int e = t; e < K; e += DK * DV / 64) {
        sm.cix[e] = reinterpret_cast<const uint16_t *>(R + hd.cidx)[e];
        sm.cvl[e] = reinterpret_cast<const float *>(R + hd.cval)[e];
    }
    __syncthreads();
    float cc[8];
    lds_read8(&sm.b.cf[8 * cg], cc, 0);
    float x[8][8];
    base_block<DK, DV>(rw, raw, sm.b, rg, cc, x);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t p0 = (uint32_t)((8 * cg + c) * DK + 8 * rg);
        const int lo = lower_bound(sm.cix, K, p0);
        for (int e = lo; e < K && sm.cix[e] < p0 + 8; ++e) {
            const int rr = (int)(sm.cix[e] - p0);
#pragma unroll
            for (int r = 0; r < 8; ++r)
                if (r == rr) x[r][c] = sm.cvl[e];
        }
    }
    if (n > 0) {
        const float *g = reinterpret_cast<const float *>(R + hd.g);
        const float *du = reinterpret_cast<const float *>(R + hd.du);
        const float *dkap = reinterpret_cast<const float *>(R + hd.dkap);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int i = 8 * rg + r;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int j = 8 * cg + c;
                float D = dkap[i] * du[j];
                for (int m = 1; m < n; ++m) D = fma_(dkap[(size_t)m * DK + i], du[(size_t)m * DV + j], D);
                x[r][c] = fma_(g[i], x[r][c], D);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        float4 *p = reinterpret_cast<float4 *>(dst + (size_t)(8 * rg + r) * DV + 8 * cg);
        p[0] = make_float4(x[r][0], x[r][1], x[r][2], x[r][3]);
        p[1] = make_float4(x[r][4], x[r][5], x[r][6], x[r][7]);
    }
}

template <int DK, int DV>
hipError_t launch_grid(void (*k)(Args), const Args &a, hipStream_t s, size_t lds = 0) {
    if (a.B == 0) return hipSuccess;
    hipLaunchKernelGGL(k, dim3((unsigned)((size_t)a.B * a.H)), dim3(DK * DV / 64), lds, s, a);
    return hipGetLastError();
}

}  // namespace

#define STQ_WIN_DISPATCH(KERNEL, LDS)                                                          \
    if (dk == 128 && dv == 128)                                                               \
        return mixed ? launch_grid<128, 128>(KERNEL<128, 128, true>, a, s, LDS)                \
                     : launch_grid<128, 128>(KERNEL<128, 128, false>, a, s, LDS);              \
    if (dk == 64 && dv == 64)                                                                 \
        return mixed ? launch_grid<64, 64>(KERNEL<64, 64, true>, a, s, LDS)                    \
                     : launch_grid<64, 64>(KERNEL<64, 64, false>, a, s, LDS);                  \
    if (dk == 128 && dv == 64)                                                                \
        return mixed ? launch_grid<128, 64>(KERNEL<128, 64, true>, a, s, LDS)                  \
                     : launch_grid<128, 64>(KERNEL<128, 64, false>, a, s, LDS);                \
    if (dk == 64 && dv == 128)                                                                \
        return mixed ? launch_grid<64, 128>(KERNEL<64, 128, true>, a, s, LDS)                  \
                     : launch_grid<64, 128>(KERNEL<64, 128, false>, a, s, LDS);                \
    return hipErrorInvalidValue;

hipError_t launch_step_win(const Args &a, int dk, int dv, bool mixed, hipStream_t s) {
    const size_t entries = (size_t)a.comps * 16;  // index, value, gated key and query per entry
    const hipError_t e = [&]() -> hipError_t { STQ_WIN_DISPATCH(k_win, entries) }();
    if (e != hipSuccess) return e;
    STQ_WIN_DISPATCH(k_win_end, 0)
}

hipError_t launch_pack_win(const Args &a, int dk, int dv, bool mixed, hipStream_t s) {
    STQ_WIN_DISPATCH(k_pack_win, 0)
}

hipError_t launch_unpack_win(const Args &a, int dk, int dv, hipStream_t s) {
    if (dk == 128 && dv == 128) return launch_grid<128, 128>(k_unpack_win<128, 128>, a, s);
    if (dk == 64 && dv == 64) return launch_grid<64, 64>(k_unpack_win<64, 64>, a, s);
    if (dk == 128 && dv == 64) return launch_grid<128, 64>(k_unpack_win<128, 64>, a, s);
    if (dk == 64 && dv == 128) return launch_grid<64, 128>(k_unpack_win<64, 128>, a, s);
    return hipErrorInvalidValue;
}

}  // namespace stq
