// Device helpers shared by the gfx950 kernels (stq_kernels.hip: per-step
// decode, pack, unpack; stq_window.hip: windowed decode).  Internal.
//
// A workgroup steps one (request, head) state of d_k x d_v at a time (the step
// kernel gives a workgroup two 4-bit heads of a request).  Thread t holds an
// 8 x 8 block: key rows 8*rg .. 8*rg+7 and value columns 8*cg .. 8*cg+7, with
// rg = t / (d_v/8) and cg = t % (d_v/8) (256 threads at d = 128, one wave at
// d = 64).  That block is the unit of every memory access: in a row of b-bit
// codes the 8 codes of one thread are b contiguous bytes, so a row piece is one
// 4 / 6 / 8 / 16-byte load.  Column sums are fma chains over the thread's 8
// rows followed by a left-to-right sum of the d_k/8 block sums in LDS; column
// and row maxima are combined the same way.  There is no matrix-core work:
// every state element is touched once against one or two vectors, so the step
// is a streaming mat-vec bound by HBM bandwidth and the VALU, not a GEMM.
//
// Arithmetic, per state (every rounding fixed so results are reproducible; the
// pages state the method in words only: STEPQuant essay, background,
// temporal-axis, spatial-axis and experiment-design paragraphs).  The stored
// state is diag(r) N diag(c); the step keeps that factored form, so the
// column scale multiplies each column once on the value side and the working
// state M'' = M / s is in units of the stored column scale:
//   s_j = c_j (1 with no column scales or c_j = 0);  is_j = RN(1/s_j)
//   g_i = RN(a_i r_i);  A_ij = RN(n_ij g_i)  (pivot row: RN(RN(a_i h_ij) is_j))
//   w_j = RN(s_j csum_i(A_ij k_i));  u_j = RN(beta RN(v_j - w_j));  u'_j = RN(u_j is_j)
//   M''_ij = fma(k_i, u'_j, A_ij);  o_j = RN(s_j csum_i(M''_ij q_i))
//   c'_j = H(RN(max_i |M''_ij| s_j));  Z_ij = RN(M''_ij RN(s_j / c'_j))
//   r'_i = Hup(RN(max_j |Z_ij| / qmax_i)) (smallest fp16 not below; fp32 row
//   scales: RN);  n'_ij = rne(Z_ij RN(1/r'_i)) -- rounding the step up keeps
//   |n'| <= qmax, so the clamp is applied only to a row whose step saturated;
//   pivot rows store H(RN(M''_ij s_j)).  Pack and the window end requantize an
//   fp32 state directly: the same with s = 1.
// csum: blocks of 8 rows as fma chains from RN(x0 y0), block sums left to right.
// Codes are offset binary (u = n + 2^(b-1)) in LSB-first row bit streams.
#pragma once

#include <hip/hip_fp16.h>

#include "stq_internal.h"

namespace stq {
namespace dev {

constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23: x + kMagic rounds x to an integer (|x| < 2^22)

__device__ __forceinline__ float fma_(float a, float b, float c) { return __builtin_fmaf(a, b, c); }

// Correctly rounded reciprocal and quotient of values with at most 11
// significant bits (fp16 values, small integers): a reciprocal estimate
// (v_rcp_f32, within an ulp) refined by one Newton step, then one correction
// of the quotient.  The exact quotient of two such values is never within
// 2^-36 (relative) of a midpoint between neighbouring floats, unless it is a
// float itself, and the refined value is within about 2^-46 of it, so its
// rounding is the correctly rounded quotient -- what an IEEE division gives.
// The residuals 1 - b r and a - b q are exact (fma of operands this short).
__device__ __forceinline__ float recip_h(float b) {
    const float r = __builtin_amdgcn_rcpf(b);
    const float e = fma_(-b, r, 1.0f);
    return fma_(e, r, r);
}
__device__ __forceinline__ float div_h(float a, float b) {
    const float y = recip_h(b);
    const float q = a * y;
    return fma_(fma_(-b, q, a), y, q);
}
// RN(a / n) for n = 2^(w-1) - 1 (7, 31 or 127) and any fp32 a: with y = RN(1/n)
// one correction gives the correctly rounded quotient (a/n is a float, or it
// is at least 2^-32 (relative) from a midpoint, n being odd and below 2^7);
// an infinite a passes through as a division would give it.
__device__ __forceinline__ float div_qmax(float a, int w) {
    const float n = (float)((1 << (w - 1)) - 1);
    const float y = w == 4 ? 1.0f / 7.0f : w == 6 ? 1.0f / 31.0f : 1.0f / 127.0f;
    const float q = a * y;
    const float c = fma_(fma_(-n, q, a), y, q);
    return __builtin_isinf(q) ? q : c;
}

// H(x): fp16 nearest-even after saturating to +-65504; returns the pattern.
__device__ __forceinline__ uint32_t h16(float x) {
    x = fminf(fmaxf(x, -65504.0f), 65504.0f);
    return (uint32_t)__half_as_ushort(__float2half_rn(x));
}
__device__ __forceinline__ float f16v(uint32_t bits) {
    return __half2float(__ushort_as_half((unsigned short)(bits & 0xffffu)));
}

// Hup(x), x >= 0: the smallest fp16 not below x, saturating at 65504.
__device__ __forceinline__ uint32_t h16up(float x) {
    uint32_t h = h16(x);
    if (f16v(h) < x && h != 0x7bffu) ++h;
    return h;
}

// Hides a value from the optimizer so byte extractions stay v_cvt_f32_ubyteN.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
    asm("" : "+v"(x));
    return x;
}

// Values whose type is chosen at run time (bf16 or fp32 inputs, fp16 or fp32
// scales) are read as the dword holding the element (ld_dword) and converted
// afterwards (dec_io, dec_scale, with the element index's parity).  No load
// then sits in a branch of its own: a load used inside a branch is waited for
// there, which would serialise a state's input loads one round trip each.
// Every such array has an even number of elements and a 4-byte aligned start,
// so the dword lies inside it.  The address is a base common to the
// workgroup (scalar registers) plus a 32-bit offset per thread, so a load
// costs one or two vector instructions of address arithmetic.
__device__ __forceinline__ uint32_t dword_off(int half, uint32_t e) {
    return half ? (e & ~1u) * 2u : e * 4u;
}
__device__ __forceinline__ uint32_t ld_dword(const void *p, int half, uint32_t e) {
    return *reinterpret_cast<const uint32_t *>(static_cast<const uint8_t *>(p) + dword_off(half, e));
}
// bf16 (if bf16) or fp32 input element of index parity `odd`: one byte
// permutation (the bf16 half moved to the top, zeros below, or the dword
// as it is)
__device__ __forceinline__ float dec_io(uint32_t d, int bf16, int odd) {
    const uint32_t sel = bf16 ? (odd ? 0x03020c0cu : 0x01000c0cu) : 0x03020100u;
    return __uint_as_float(__builtin_amdgcn_perm(d, d, sel));
}
// fp16 (if f16) or fp32 scale of index parity `odd`
__device__ __forceinline__ float dec_scale(uint32_t d, int f16, int odd) {
    return f16 ? f16v(odd ? d >> 16 : d) : __uint_as_float(d);
}

// The per-state inputs thread t reads, for key row t (t < d_k) and value
// column t (t < d_v), as raw dwords.  Threads past d_k or d_v read element 0
// and do not use it, so the loads need no branch.
struct Inputs {
    float a, beta;
    uint32_t r, k, q;  // key row t: row scale, key, query
    uint32_t c, v;     // value column t: column scale, value
    uint32_t nr, nc;   // lagged scales: next row scale of row t % d_k, next
                       // column scale of column t % d_v (else unused)
};

// A use of every input dword on all threads, placed once they have been
// used: the loads then cannot be moved into the branches that use them (which
// would issue them late, behind loads meant to be in flight longer).
__device__ __forceinline__ void keep_inputs(const Inputs &p) {
    asm volatile("" ::"v"(p.a), "v"(p.beta), "v"(p.r), "v"(p.k), "v"(p.q), "v"(p.c), "v"(p.v));
}
__device__ __forceinline__ void keep_lagged(const Inputs &p) {
    asm volatile("" ::"v"(p.nr), "v"(p.nc));
}

template <int DK, int DV, bool LAG = false>
__device__ __forceinline__ void fetch_inputs(const Args &A, const HeadDesc &hd, const uint8_t *R, size_t unit,
                                             int t, Inputs &p) {
    const uint32_t tk = t < DK ? t : 0, tv = t < DV ? t : 0;
    p.nr = p.nc = 0;
    if (LAG) {
        // a head without these sections has offset 0 here: inside its region
        p.nr = ld_dword(R + hd.nrs, A.rs16, (uint32_t)t % DK);
        p.nc = ld_dword(R + hd.ncs, 1, (uint32_t)t % DV);
    }
    p.beta = A.beta[unit];
    // the state's rows of the inputs (uniform), then one offset per thread
    const size_t es = A.io_bf16 ? 2 : 4;
    const uint8_t *kb = static_cast<const uint8_t *>(A.k) + unit * (DK * es);
    const uint8_t *qb = static_cast<const uint8_t *>(A.q) + unit * (DK * es);
    const uint8_t *vb = static_cast<const uint8_t *>(A.v) + unit * (DV * es);
    const float *ab = A.a + (A.gate_vec ? unit * DK : unit);
    p.a = ab[A.gate_vec ? tk : 0u];
    // a head without scales has offset 0 here: still inside its region
    p.r = ld_dword(R + hd.rs, A.rs16, tk);
    p.k = ld_dword(kb, A.io_bf16, tk);
    p.q = ld_dword(qb, A.io_bf16, tk);
    p.c = ld_dword(R + hd.cs, 1, tv);
    p.v = ld_dword(vb, A.io_bf16, tv);
}

// A head's width and quantized-row count share one descriptor dword; reading
// the dword keeps the load on the scalar unit (no 16-bit scalar loads).
__device__ __forceinline__ uint32_t head_wq(const HeadDesc &hd) {
    static_assert(offsetof(HeadDesc, wq) == 44, "width and nquant share the 12th dword");
    return hd.wq;
}
__device__ __forceinline__ int head_width(const HeadDesc &hd) { return (int)(head_wq(hd) & 0xffffu); }
__device__ __forceinline__ int head_nquant(const HeadDesc &hd) { return (int)(head_wq(hd) >> 16); }

// The piece of a row owned by column group cg: 8 codes of w bits = w bytes.
__device__ __forceinline__ uint4 load_piece(const uint8_t *row, int cg, int w) {
    uint4 r = make_uint4(0, 0, 0, 0);
    if (w == 4) {
        r.x = *reinterpret_cast<const uint32_t *>(row + 4 * cg);
    } else if (w == 8) {
        const uint2 v = *reinterpret_cast<const uint2 *>(row + 8 * cg);
        r.x = v.x; r.y = v.y;
    } else if (w == 6) {
        // 6 bytes at a 2-byte aligned offset: the two dwords around them,
        // shifted (they stay inside the row: 6*cg + 6 <= row bytes, and the
        // aligned start is at most 2 bytes before the piece)
        const uint32_t off = 6u * (uint32_t)cg;
        const uint32_t *q = reinterpret_cast<const uint32_t *>(row + (off & ~3u));
        const uint32_t lo = q[0], hi = q[1];
        const uint32_t sh = (off & 3u) * 8u;  // 0 or 16
        r.x = __builtin_amdgcn_alignbit(hi, lo, sh);
        r.y = hi >> sh;                       // bits above 15 are not read
    } else {
        r = *reinterpret_cast<const uint4 *>(row + 16 * cg);
    }
    return r;
}

__device__ __forceinline__ void store_piece(uint8_t *row, int cg, int w, uint4 r) {
    if (w == 4) {
        *reinterpret_cast<uint32_t *>(row + 4 * cg) = r.x;
    } else if (w == 8) {
        *reinterpret_cast<uint2 *>(row + 8 * cg) = make_uint2(r.x, r.y);
    } else if (w == 6) {
        uint16_t *p = reinterpret_cast<uint16_t *>(row + 6 * cg);
        p[0] = (uint16_t)(r.x & 0xffffu);
        p[1] = (uint16_t)(r.x >> 16);
        p[2] = (uint16_t)(r.y & 0xffffu);
    } else {
        *reinterpret_cast<uint4 *>(row + 16 * cg) = r;
    }
}

// Unsigned (offset-binary) codes of a piece as floats.  For 4-bit pieces the
// odd codes come out multiplied by 16 (their nibble stays in place); the
// caller scales them by g/16, which is exact.
__device__ __forceinline__ void codes_f(uint4 r, int w, float u[8]) {
    if (w == 4) {
        const uint32_t lo = opaque(r.x & 0x0F0F0F0Fu), hi = opaque(r.x & 0xF0F0F0F0u);
        u[0] = (float)(lo & 0xffu);         u[1] = (float)(hi & 0xffu);
        u[2] = (float)((lo >> 8) & 0xffu);  u[3] = (float)((hi >> 8) & 0xffu);
        u[4] = (float)((lo >> 16) & 0xffu); u[5] = (float)((hi >> 16) & 0xffu);
        u[6] = (float)(lo >> 24);           u[7] = (float)(hi >> 24);
    } else if (w == 8) {
        const uint32_t x = opaque(r.x), y = opaque(r.y);
        u[0] = (float)(x & 0xffu);         u[1] = (float)((x >> 8) & 0xffu);
        u[2] = (float)((x >> 16) & 0xffu); u[3] = (float)(x >> 24);
        u[4] = (float)(y & 0xffu);         u[5] = (float)((y >> 8) & 0xffu);
        u[6] = (float)((y >> 16) & 0xffu); u[7] = (float)(y >> 24);
    } else {  // 6: codes 0-4 in x, code 5 across x and y, codes 6-7 in y
        const uint32_t x = r.x, y = r.y;
        u[0] = (float)(x & 63u);
        u[1] = (float)((x >> 6) & 63u);
        u[2] = (float)((x >> 12) & 63u);
        u[3] = (float)((x >> 18) & 63u);
        u[4] = (float)((x >> 24) & 63u);
        u[5] = (float)(__builtin_amdgcn_alignbit(y, x, 30) & 63u);
        u[6] = (float)((y >> 4) & 63u);
        u[7] = (float)((y >> 10) & 63u);
    }
}

// Codes scaled by the row step: RN((u - 2^(w-1)) * g), with u, g and the
// offset term exact, so one fma rounds once.  g16 = g / 16, nog = -2^(w-1) g.
__device__ __forceinline__ void dequant_row(uint4 raw, int w, float g, float g16, float nog, float x[8]) {
    float u[8];
    codes_f(raw, w, u);
    if (w == 4) {
#pragma unroll
        for (int c = 0; c < 8; c += 2) {
            x[c] = fma_(u[c], g, nog);
            x[c + 1] = fma_(u[c + 1], g16, nog);
        }
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) x[c] = fma_(u[c], g, nog);
    }
}

// Pack 8 quantized values y = 1.5*2^23 + 2^(w-1) + n into a piece: the low
// byte of each pattern is the offset-binary code (no carry out of the field).
__device__ __forceinline__ uint4 pack_codes(const float y[8], int w) {
    uint4 r = make_uint4(0, 0, 0, 0);
    uint32_t b[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) b[c] = __float_as_uint(y[c]);
    if (w == 4) {
        // byte 0 of each pair word = two nibbles, byte 1 = 0
        const uint32_t p01 = (b[1] << 4) | b[0], p23 = (b[3] << 4) | b[2];
        const uint32_t p45 = (b[5] << 4) | b[4], p67 = (b[7] << 4) | b[6];
        r.x = __builtin_amdgcn_perm(p23, p01, 0x0c0c0400u) | __builtin_amdgcn_perm(p67, p45, 0x04000c0cu);
    } else if (w == 8) {
        // byte 1 of each pattern is 0, so a shifted or keeps two clean bytes
        const uint32_t p01 = (b[1] << 8) | b[0], p23 = (b[3] << 8) | b[2];
        const uint32_t p45 = (b[5] << 8) | b[4], p67 = (b[7] << 8) | b[6];
        r.x = __builtin_amdgcn_perm(p23, p01, 0x05040100u);
        r.y = __builtin_amdgcn_perm(p67, p45, 0x05040100u);
    } else {  // 6
        uint32_t u[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) u[c] = b[c] & 63u;
        r.x = u[0] | (u[1] << 6) | (u[2] << 12) | (u[3] << 18) | (u[4] << 24) | (u[5] << 30);
        r.y = (u[5] >> 2) | (u[6] << 4) | (u[7] << 10);
    }
    return r;
}

// LDS of one workgroup.  The per-thread partials are stored element-major,
// thread-minor ([c][t], with t = rg * d_v/8 + cg): each write of the 64 lanes of
// a wave is then one contiguous run, and the 4-float pad spreads the combining
// reads (a column's partials sit at [j % 8][rg * d_v/8 + j / 8]; a row's at
// [i % 8][i / 8 * d_v/8 + cg]) over the banks.
template <int DK, int DV>
struct alignas(16) Lds {
    static constexpr int NT = DK * DV / 64;
    static constexpr int NTP = NT + 4;
    float colp[8][NTP];         // column partial sums: [c][t]
    union {
        float colm[8][NTP];     // column partial maxima: [c][t]
        float rowm[8][NTP];     // row partial maxima: [r][t] (after the column maxima are used)
    };
    float g[DK];                // per key row: gated row step RN(a r)
    float g16[DK];              //   g / 16
    float nog[DK];              //   -2^(w-1) g
    float af[DK];               //   gate
    float om[DK];               //   row-impact weight (1 without scores)
    float kf[DK], qf[DK];       //   k and q as fp32
    float cf[DV];               // column factor s (the column scale, or 1)
    float isf[DV];              // RN(1 / s)
    float u[DV];                // u' = RN(beta (v - w) / s)
    float ic[DV];               // RN(s / c') (pack: RN(1 / c'))
    float ir[DK];               // 1 / r'; negated when the row step saturated
};

// Left-to-right sum of the d_k/8 block partials of column j.
template <int DK, int DV>
__device__ __forceinline__ float col_sum(const Lds<DK, DV> &sm, int j) {
    constexpr int CG = DV / 8, RG = DK / 8;
    const float *p = &sm.colp[j & 7][j >> 3];
    float s = p[0];
#pragma unroll
    for (int g = 1; g < RG; ++g) s = s + p[g * CG];
    return s;
}

template <int DK, int DV>
__device__ __forceinline__ float col_max(const Lds<DK, DV> &sm, int j) {
    constexpr int CG = DV / 8, RG = DK / 8;
    const float *p = &sm.colm[j & 7][j >> 3];
    float m = p[0];
#pragma unroll
    for (int g = 1; g < RG; ++g) m = fmaxf(m, p[g * CG]);
    return m;
}

// The d_v/8 partials of a row are contiguous and 16-byte aligned (rows of
// the array are NTP = NT + 4 floats, a multiple of 4): read four at a time.
template <int DK, int DV>
__device__ __forceinline__ float row_max(const Lds<DK, DV> &sm, int i) {
    constexpr int CG = DV / 8;
    static_assert(CG % 4 == 0 && Lds<DK, DV>::NTP % 4 == 0, "row partials in 16-byte groups");
    const float4 *p = reinterpret_cast<const float4 *>(&sm.rowm[i & 7][(i >> 3) * CG]);
    float v[CG];
#pragma unroll
    for (int g = 0; g < CG / 4; ++g) {
        const float4 f = p[g];
        v[4 * g] = f.x; v[4 * g + 1] = f.y; v[4 * g + 2] = f.z; v[4 * g + 3] = f.w;
    }
    float m = v[0];
#pragma unroll
    for (int g = 1; g < CG; ++g) m = fmaxf(m, v[g]);
    return m;
}

// Per-thread view of one state during a step / pack.
struct Rows {
    int w[8];        // width of each of the thread's rows
    uint32_t ro[8];  // byte offset of each row inside the head region
    uint32_t m8;     // kW4P: pivot bits of the thread's 8 rows (w and ro unused)
    uint32_t base;   // kW4P: byte offset of the thread's first row
};

// W: the head's uniform row width (32: fp32 rows), or 0 / kW4P for per-row
// widths.
template <int W>
constexpr bool per_row() { return W == 0 || W == kW4P; }

// kW4P heads: the pivot bits of key rows [32 j, 32 j + 32) for a per-thread j.
__device__ __forceinline__ uint32_t pivot_word(const HeadDesc &hd, int j) {
    const uint32_t m0 = hd.pmask[0], m1 = hd.pmask[1], m2 = hd.pmask[2], m3 = hd.pmask[3];
    return j == 0 ? m0 : j == 1 ? m1 : j == 2 ? m2 : m3;
}

// kW4P heads: the pivot bits of the thread's rows 8 rg .. 8 rg + 7, and the
// byte offset of row 8 rg (4-bit rows take d_v/2 bytes, pivot rows 2 d_v).
template <int DV>
__device__ __forceinline__ uint32_t pivot_block(const HeadDesc &hd, int rg, uint32_t &base) {
    const int i = 8 * rg, j = i >> 5, sh = i & 31;
    const uint32_t wj = pivot_word(hd, j);
    uint32_t before = __builtin_popcount(wj & ((1u << sh) - 1u));
#pragma unroll
    for (int k = 0; k < 3; ++k) before += k < j ? __builtin_popcount(hd.pmask[k]) : 0u;
    base = (uint32_t)i * (DV / 2) + before * (3 * DV / 2);
    return (wj >> sh) & 0xffu;
}

template <int DV, int W>
__device__ __forceinline__ void row_geometry(const Args &A, const HeadDesc &hd, int rg, Rows &rw) {
    if (W == kW4P) {
        // kept as a mask and one offset; row_w and row_o derive the rest
        rw.m8 = pivot_block<DV>(hd, rg, rw.base);
        return;
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        if (!per_row<W>()) {
            rw.w[r] = W;
            rw.ro[r] = (uint32_t)(8 * rg + r) * (uint32_t)(DV * W / 8);
        } else {
            const uint32_t e = A.rows[hd.rows + 8 * rg + r];
            rw.w[r] = (int)row_width(e);
            rw.ro[r] = row_off(e);
        }
    }
}

// Width and byte offset of the thread's row r.
template <int W>
__device__ __forceinline__ int row_w(const Rows &rw, int r) {
    return W == kW4P ? ((rw.m8 >> r) & 1u ? 16 : 4) : rw.w[r];
}
template <int DV, int W>
__device__ __forceinline__ uint32_t row_o(const Rows &rw, int r) {
    if (W != kW4P) return rw.ro[r];
    const uint32_t piv_before = __builtin_popcount(rw.m8 & ((1u << r) - 1u));
    return rw.base + (uint32_t)r * (DV / 2) + piv_before * (3 * DV / 2);
}

// Width of key row i of the head (uniform width, the pivot mask or the row table).
template <int W>
__device__ __forceinline__ int width_of(const Args &A, const HeadDesc &hd, int i) {
    if (W == kW4P) return (pivot_word(hd, i >> 5) >> (i & 31)) & 1u ? 16 : 4;
    return !per_row<W>() ? W : (int)row_width(A.rows[hd.rows + i]);
}

// Whether the head has quantized rows: known from the width unless rows differ.
template <int W>
__device__ __forceinline__ bool has_quant(const HeadDesc &hd) {
    return (W == 16 || W == 32) ? false : (!per_row<W>() ? true : head_nquant(hd) > 0);
}

template <int N>
__device__ __forceinline__ void lds_read8(const float *p, float (&out)[N], int o) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    out[o + 0] = a.x; out[o + 1] = a.y; out[o + 2] = a.z; out[o + 3] = a.w;
    out[o + 4] = b.x; out[o + 5] = b.y; out[o + 6] = b.z; out[o + 7] = b.w;
}

__device__ __forceinline__ uint4 pivot_piece(const float (&x)[8]) {
    uint4 p;
    p.x = h16(x[0]) | (h16(x[1]) << 16);
    p.y = h16(x[2]) | (h16(x[3]) << 16);
    p.z = h16(x[4]) | (h16(x[5]) << 16);
    p.w = h16(x[6]) | (h16(x[7]) << 16);
    return p;
}

// A pivot row piece of the working state (SCALED: in units of the column
// factor s): the fp16 of RN(x s).
template <bool SCALED>
__device__ __forceinline__ uint4 pivot_piece_s(const float (&x)[8], const float (&s)[8]) {
    if (!SCALED) return pivot_piece(x);
    float y[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) y[c] = x[c] * s[c];
    return pivot_piece(y);
}

// Quantize one row of 8 values with 1/r' = ir and store the piece.
template <bool CLAMP>
__device__ __forceinline__ void quant_row(uint8_t *row, int cg, int w, float ir, const float (&x)[8]) {
    const float off = (float)(1 << (w - 1));
    const float mg = kMagic + off;
    float y[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        y[c] = fma_(x[c], ir, mg);
        if (CLAMP) y[c] = fminf(fmaxf(y[c], mg - (off - 1.0f)), mg + (off - 1.0f));
    }
    store_piece(row, cg, w, pack_codes(y, w));
}

// Column scales, row scales, codes and pivots of x (the thread's 8x8 block of
// the fp32 state) written back into the head region R.  SCALED: x is in units
// of the column factor s in sm.cf (the step's working state); otherwise x is
// the state itself (pack, window end).  If emit_o, the column partial sums of
// o are already in sm.colp and o is combined and stored in the same LDS round
// as the column maxima.  fw (kW4P heads, uniform over the wave): no block of
// the wave holds a pivot row, so every row is 4-bit and rows follow each
// other at d_v/2 bytes from rw.base.
template <int DK, int DV, int W, bool SCALED, bool IMP = false>
__device__ __forceinline__ void requant_store(const Args &A, const HeadDesc &hd, uint8_t *R,
                                              const Rows &rw, float (&x)[8][8], Lds<DK, DV> &sm,
                                              int t, int rg, int cg, bool emit_o, size_t unit,
                                              bool fw = false) {
    const bool quant = has_quant<W>(hd);
    const bool cs = quant && A.cs16;
    // column maxima over quantized rows (with row-impact weights: of w_i |x|;
    // IMP instantiations only, the weighted loop costs registers)
    if (IMP && cs) {
        float om[8];
        lds_read8(&sm.om[8 * rg], om, 0);
        const bool all_q = !per_row<W>() || fw;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float m = 0.0f;
#pragma unroll
            for (int r = 0; r < 8; ++r)
                if (all_q || row_w<W>(rw, r) != 16) m = fmaxf(m, om[r] * fabsf(x[r][c]));
            sm.colm[c][t] = m;
        }
    } else if (cs && (!per_row<W>() || fw)) {
        // every row quantized: two elements per max3
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float m = 0.0f;
#pragma unroll
            for (int r = 0; r < 8; ++r) m = fmaxf(m, fabsf(x[r][c]));
            sm.colm[c][t] = m;
        }
    } else if (cs) {
        // rows of differing widths: a pair of rows that holds no pivot row in
        // any block of the wave (a wave-uniform test) takes the unmasked
        // max3, the others a per-lane test
        uint32_t wm = 0u;
#pragma unroll
        for (int r = 0; r < 8; ++r) wm |= (__any(row_w<W>(rw, r) == 16) ? 1u : 0u) << r;
        float m[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) m[c] = 0.0f;
#pragma unroll
        for (int r = 0; r < 8; r += 2) {
            if (((wm >> r) & 3u) == 0u) {
#pragma unroll
                for (int c = 0; c < 8; ++c) m[c] = fmaxf(m[c], fmaxf(fabsf(x[r][c]), fabsf(x[r + 1][c])));
            } else {
                const bool q0 = row_w<W>(rw, r) != 16, q1 = row_w<W>(rw, r + 1) != 16;
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    if (q0) m[c] = fmaxf(m[c], fabsf(x[r][c]));
                    if (q1) m[c] = fmaxf(m[c], fabsf(x[r + 1][c]));
                }
            }
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) sm.colm[c][t] = m[c];
    }
    if (cs || emit_o) __syncthreads();
    // o of column t, and the new scale of column tc: with at least 2 d_v
    // threads, threads [0, d_v) combine o while threads [d_v, 2 d_v) form the
    // scales, so the two serial combines run side by side
    constexpr int NT = DK * DV / 64;
    if (emit_o && t < DV) {
        const float op = col_sum<DK, DV>(sm, t);
        A.o[unit * DV + t] = SCALED ? sm.cf[t] * op : op;
    }
    const int tc = (emit_o && NT >= 2 * DV) ? t - DV : t;
    if (tc >= 0 && tc < DV) {
        float ic = 1.0f;
        if (cs) {
            const float C = col_max<DK, DV>(sm, tc);
            const float sj = SCALED ? sm.cf[tc] : 1.0f;
            const float Cs = SCALED ? C * sj : C;
            // lagged-scale layouts record the refit statistics
            if (A.lagged) reinterpret_cast<float *>(R + hd.scs)[tc] = Cs;
            const uint32_t hc = h16(Cs);
            const float cv = f16v(hc);
            ic = cv > 0.0f ? div_h(sj, cv) : 0.0f;  // sj and cv are fp16 values
            reinterpret_cast<uint16_t *>(R + hd.cs)[tc] = (uint16_t)hc;
        }
        sm.ic[tc] = ic;
    }
    if (!quant) {
        // all rows are FP16 pivots (or fp32 rows, stored as they are): store and finish
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if (W == 32) {
                float4 *p = reinterpret_cast<float4 *>(R + row_o<DV, W>(rw, r) + 32 * cg);
                p[0] = make_float4(x[r][0], x[r][1], x[r][2], x[r][3]);
                p[1] = make_float4(x[r][4], x[r][5], x[r][6], x[r][7]);
            } else {
                store_piece(R + row_o<DV, W>(rw, r), cg, 16, pivot_piece(x[r]));
            }
        }
        return;
    }
    __syncthreads();
    float icc[8];
    lds_read8(&sm.ic[8 * cg], icc, 0);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        float m = 0.0f;
        if (fw || row_w<W>(rw, r) != 16) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float z = x[r][c] * icc[c];
                x[r][c] = z;
                m = fmaxf(m, fabsf(z));
            }
        }
        sm.rowm[r][t] = m;
    }
    __syncthreads();
    if (t < DK) {
        const int w = width_of<W>(A, hd, t);
        float ir = 0.0f, rv = 0.0f;
        uint32_t rh = 0;  // fp16 pattern of the row step (0 for a pivot row)
        bool sat = false;
        if (w != 16) {
            const float Rm = row_max<DK, DV>(sm, t);
            if (A.lagged) reinterpret_cast<float *>(R + hd.srs)[t] = Rm;
            const float rq = div_qmax(Rm, w);
            if (A.rs16) {
                rh = h16up(rq);
                rv = f16v(rh);
                sat = rq > 65504.0f;
                ir = rv > 0.0f ? recip_h(rv) : 0.0f;  // rv is an fp16 value
            } else {
                rv = rq;
                ir = rv > 0.0f ? 1.0f / rv : 0.0f;
                if (__builtin_isinf(ir)) ir = 0.0f;
            }
        }
        if (A.rs16) reinterpret_cast<uint16_t *>(R + hd.rs)[t] = (uint16_t)rh;
        else reinterpret_cast<float *>(R + hd.rs)[t] = rv;
        sm.ir[t] = sat ? -ir : ir;
    }
    __syncthreads();
    float irr[8];
    lds_read8(&sm.ir[8 * rg], irr, 0);
    // pivot rows among quantized rows (per-row heads only) store H(RN(x s))
    float scc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) scc[c] = 1.0f;
    if (SCALED && per_row<W>()) lds_read8(&sm.cf[8 * cg], scc, 0);
    // a negative 1/r' marks a saturated row (1/r' is +0 or positive
    // otherwise); the OR of the eight sign bits finds one in four or3
    // operations (a flag per row costs a compare and a select each)
    uint32_t irsign = __float_as_uint(irr[0]);
#pragma unroll
    for (int r = 1; r < 8; ++r) irsign |= __float_as_uint(irr[r]);
    if (__builtin_expect(__any((int32_t)irsign < 0), 0)) {
        // a row step saturated at 65504: clamp codes to +-qmax
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if (row_w<W>(rw, r) == 16) store_piece(R + row_o<DV, W>(rw, r), cg, 16, pivot_piece_s<SCALED>(x[r], scc));
            else quant_row<true>(R + row_o<DV, W>(rw, r), cg, row_w<W>(rw, r), fabsf(irr[r]), x[r]);
        }
    } else if (W == kW4P && fw) {
#pragma unroll
        for (int r = 0; r < 8; ++r) quant_row<false>(R + rw.base + (uint32_t)r * (DV / 2), cg, 4, irr[r], x[r]);
    } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            if (row_w<W>(rw, r) == 16) store_piece(R + row_o<DV, W>(rw, r), cg, 16, pivot_piece_s<SCALED>(x[r], scc));
            else quant_row<false>(R + row_o<DV, W>(rw, r), cg, row_w<W>(rw, r), irr[r], x[r]);
        }
    }
}

}  // namespace dev
}  // namespace stq
