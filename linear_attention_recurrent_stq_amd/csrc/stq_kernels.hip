// HIP kernels for gfx950: decode step, pack, unpack and pool init of the
// quantized recurrent state.
//
// One workgroup owns one (request, head) state of d_k x d_v.  Thread t holds an
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
// temporal-axis, spatial-axis and experiment-design paragraphs):
//   g_i = RN(a_i r_i);  A_ij = RN(RN(n_ij g_i) c_j)  (pivot row: RN(a_i h_ij))
//   w_j = csum_i(A_ij k_i);  u_j = RN(beta RN(v_j - w_j))
//   M_ij = fma(k_i, u_j, A_ij);  o_j = csum_i(M_ij q_i)
//   c'_j = H(max_i |M_ij|);  Z_ij = RN(M_ij RN(1/c'_j))
//   r'_i = H(RN(max_j |Z_ij| / qmax_i));  n'_ij = clamp(rne(Z_ij RN(1/r'_i)))
// csum: blocks of 8 rows as fma chains from RN(x0 y0), block sums left to right.
// Codes are offset binary (u = n + 2^(b-1)) in LSB-first row bit streams.
#include <hip/hip_fp16.h>

#include "stq_internal.h"

namespace stq {
namespace {

constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23: x + kMagic rounds x to an integer (|x| < 2^22)

__device__ __forceinline__ float fma_(float a, float b, float c) { return __builtin_fmaf(a, b, c); }

// H(x): fp16 nearest-even after saturating to +-65504; returns the pattern.
__device__ __forceinline__ uint32_t h16(float x) {
    x = fminf(fmaxf(x, -65504.0f), 65504.0f);
    return (uint32_t)__half_as_ushort(__float2half_rn(x));
}
__device__ __forceinline__ float f16v(uint32_t bits) {
    return __half2float(__ushort_as_half((unsigned short)(bits & 0xffffu)));
}

// 8 consecutive io values (bf16 or fp32) starting at element e (e % 8 == 0).
__device__ __forceinline__ void load8(const void *p, int bf16, size_t e, float out[8]) {
    if (bf16) {
        const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p) + e);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            out[2 * c] = __uint_as_float(w[c] << 16);
            out[2 * c + 1] = __uint_as_float(w[c] & 0xffff0000u);
        }
    } else {
        const float4 *f = reinterpret_cast<const float4 *>(static_cast<const float *>(p) + e);
        const float4 a = f[0], b = f[1];
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
        out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    }
}

__device__ __forceinline__ float load1(const void *p, int bf16, size_t e) {
    if (bf16) return __uint_as_float((uint32_t)(static_cast<const uint16_t *>(p)[e]) << 16);
    return static_cast<const float *>(p)[e];
}

// The piece of a row owned by column group cg: 8 codes of w bits = w bytes.
__device__ __forceinline__ uint4 load_piece(const uint8_t *row, int cg, int w) {
    uint4 r = make_uint4(0, 0, 0, 0);
    if (w == 4) {
        r.x = *reinterpret_cast<const uint32_t *>(row + 4 * cg);
    } else if (w == 8) {
        const uint2 v = *reinterpret_cast<const uint2 *>(row + 8 * cg);
        r.x = v.x; r.y = v.y;
    } else if (w == 6) {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(row + 6 * cg);
        r.x = (uint32_t)p[0] | ((uint32_t)p[1] << 16);
        r.y = p[2];
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

// Unsigned (offset-binary) codes of a piece as floats.
__device__ __forceinline__ void codes_f(uint4 r, int w, float u[8]) {
    if (w == 4) {
        const uint32_t lo = r.x & 0x0F0F0F0Fu, hi = (r.x >> 4) & 0x0F0F0F0Fu;
        u[0] = (float)(lo & 0xffu);         u[1] = (float)(hi & 0xffu);
        u[2] = (float)((lo >> 8) & 0xffu);  u[3] = (float)((hi >> 8) & 0xffu);
        u[4] = (float)((lo >> 16) & 0xffu); u[5] = (float)((hi >> 16) & 0xffu);
        u[6] = (float)(lo >> 24);           u[7] = (float)(hi >> 24);
    } else if (w == 8) {
        u[0] = (float)(r.x & 0xffu);         u[1] = (float)((r.x >> 8) & 0xffu);
        u[2] = (float)((r.x >> 16) & 0xffu); u[3] = (float)(r.x >> 24);
        u[4] = (float)(r.y & 0xffu);         u[5] = (float)((r.y >> 8) & 0xffu);
        u[6] = (float)((r.y >> 16) & 0xffu); u[7] = (float)(r.y >> 24);
    } else {  // 6
        const uint64_t v = (uint64_t)r.x | ((uint64_t)r.y << 32);
#pragma unroll
        for (int c = 0; c < 8; ++c) u[c] = (float)(uint32_t)((v >> (6 * c)) & 63u);
    }
}

// Pack 8 quantized values y (kMagic + 2^(w-1) + n, clamped) into a piece.
__device__ __forceinline__ uint4 pack_codes(const float y[8], int w) {
    uint4 r = make_uint4(0, 0, 0, 0);
    uint32_t u[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) u[c] = __float_as_uint(y[c]) & ((1u << w) - 1u);
    if (w == 4) {
        r.x = u[0] | (u[1] << 4) | (u[2] << 8) | (u[3] << 12) | (u[4] << 16) | (u[5] << 20) |
              (u[6] << 24) | (u[7] << 28);
    } else if (w == 8) {
        r.x = u[0] | (u[1] << 8) | (u[2] << 16) | (u[3] << 24);
        r.y = u[4] | (u[5] << 8) | (u[6] << 16) | (u[7] << 24);
    } else {  // 6
        r.x = u[0] | (u[1] << 6) | (u[2] << 12) | (u[3] << 18) | (u[4] << 24) | (u[5] << 30);
        r.y = (u[5] >> 2) | (u[6] << 4) | (u[7] << 10);
    }
    return r;
}

template <int DK, int DV>
struct Lds {
    float colp[DK / 8][DV];  // column partial sums
    float colm[DK / 8][DV];  // column partial maxima
    float rowm[DV / 8][DK];  // row partial maxima
    float u[DV];
    float ic[DV];
    float ir[DK];
};

// Per-thread view of one state during a step / pack.
struct Rows {
    int w[8];        // width of each of the thread's rows
    uint32_t ro[8];  // byte offset of each row inside the head region
};

template <int DV, int W>
__device__ __forceinline__ void row_geometry(const Args &A, const HeadDesc &hd, int rg, Rows &rw) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        if (W) {
            rw.w[r] = W;
            rw.ro[r] = (uint32_t)(8 * rg + r) * (uint32_t)(DV * W / 8);
        } else {
            const uint32_t e = A.rows[hd.rows + 8 * rg + r];
            rw.w[r] = (int)row_width(e);
            rw.ro[r] = row_off(e);
        }
    }
}

// Width of key row i of the head (uniform width or the row table).
template <int W>
__device__ __forceinline__ int width_of(const Args &A, const HeadDesc &hd, int i) {
    return W ? W : (int)row_width(A.rows[hd.rows + i]);
}

// Column scales, row scales, codes and pivots of x (the thread's 8x8 block of
// the fp32 state) written back into the head region R.  If emit_o, the column
// partial sums of o are already in sm.colp and o is combined and stored in the
// same LDS round as the column maxima.
template <int DK, int DV, int W>
__device__ __forceinline__ void requant_store(const Args &A, const HeadDesc &hd, uint8_t *R,
                                              const Rows &rw, float (&x)[8][8], Lds<DK, DV> &sm,
                                              int t, int rg, int cg, bool emit_o, size_t unit) {
    constexpr int RG = DK / 8, CG = DV / 8;
    const bool quant = hd.nquant > 0;
    const bool cs = quant && A.cs16;
    // column maxima over quantized rows
    if (cs) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float m = 0.0f;
#pragma unroll
            for (int r = 0; r < 8; ++r)
                if (rw.w[r] != 16) m = fmaxf(m, fabsf(x[r][c]));
            sm.colm[rg][8 * cg + c] = m;
        }
    }
    if (cs || emit_o) __syncthreads();
    if (t < DV) {
        if (emit_o) {
            float o = sm.colp[0][t];
#pragma unroll
            for (int g = 1; g < RG; ++g) o = o + sm.colp[g][t];
            A.o[unit * DV + t] = o;
        }
        float ic = 1.0f;
        if (cs) {
            float C = sm.colm[0][t];
#pragma unroll
            for (int g = 1; g < RG; ++g) C = fmaxf(C, sm.colm[g][t]);
            const uint32_t hc = h16(C);
            const float cv = f16v(hc);
            ic = cv > 0.0f ? 1.0f / cv : 0.0f;
            reinterpret_cast<uint16_t *>(R + hd.cs)[t] = (uint16_t)hc;
        }
        sm.ic[t] = ic;
    }
    if (!quant) {
        // all rows are FP16 pivots: store and finish
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            uint4 p;
            p.x = h16(x[r][0]) | (h16(x[r][1]) << 16);
            p.y = h16(x[r][2]) | (h16(x[r][3]) << 16);
            p.z = h16(x[r][4]) | (h16(x[r][5]) << 16);
            p.w = h16(x[r][6]) | (h16(x[r][7]) << 16);
            store_piece(R + rw.ro[r], cg, 16, p);
        }
        return;
    }
    __syncthreads();
    float icc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) icc[c] = sm.ic[8 * cg + c];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        float m = 0.0f;
        if (rw.w[r] != 16) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float z = x[r][c] * icc[c];
                x[r][c] = z;
                m = fmaxf(m, fabsf(z));
            }
        }
        sm.rowm[cg][8 * rg + r] = m;
    }
    __syncthreads();
    if (t < DK) {
        const int w = width_of<W>(A, hd, t);
        float ir = 0.0f;
        float rv = 0.0f;
        if (w != 16) {
            float Rm = sm.rowm[0][t];
#pragma unroll
            for (int g = 1; g < CG; ++g) Rm = fmaxf(Rm, sm.rowm[g][t]);
            const float rq = Rm / (float)((1 << (w - 1)) - 1);
            rv = A.rs16 ? f16v(h16(rq)) : rq;
            ir = rv > 0.0f ? 1.0f / rv : 0.0f;
        }
        if (A.rs16) reinterpret_cast<uint16_t *>(R + hd.rs)[t] = (uint16_t)h16(rv);
        else reinterpret_cast<float *>(R + hd.rs)[t] = rv;
        sm.ir[t] = ir;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int w = rw.w[r];
        uint4 p;
        if (w == 16) {
            p.x = h16(x[r][0]) | (h16(x[r][1]) << 16);
            p.y = h16(x[r][2]) | (h16(x[r][3]) << 16);
            p.z = h16(x[r][4]) | (h16(x[r][5]) << 16);
            p.w = h16(x[r][6]) | (h16(x[r][7]) << 16);
        } else {
            const float irr = sm.ir[8 * rg + r];
            const float off = (float)(1 << (w - 1));
            const float mg = kMagic + off;
            const float lo = mg - (off - 1.0f), hi = mg + (off - 1.0f);
            float y[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) y[c] = fminf(fmaxf(fma_(x[r][c], irr, mg), lo), hi);
            p = pack_codes(y, w);
        }
        store_piece(R + rw.ro[r], cg, w, p);
    }
}

// ----------------------------------------------------------------- step

template <int DK, int DV, int W>
__device__ __forceinline__ void step_tile(const Args &A, const HeadDesc &hd, uint8_t *R,
                                          Lds<DK, DV> &sm, int t, int rg, int cg, size_t unit,
                                          const float (&kk)[8], const float (&qq)[8],
                                          const float (&aa)[8], float beta, float vv) {
    constexpr int RG = DK / 8;
    Rows rw;
    row_geometry<DV, W>(A, hd, rg, rw);
    uint4 raw[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) raw[r] = load_piece(R + rw.ro[r], cg, rw.w[r]);
    float rr[8], cc[8];
    const bool quant = hd.nquant > 0;
    if (quant) {
        if (A.rs16) {
            const uint4 s = *reinterpret_cast<const uint4 *>(R + hd.rs + 16 * rg);
            const uint32_t sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) { rr[2 * c] = f16v(sv[c]); rr[2 * c + 1] = f16v(sv[c] >> 16); }
        } else {
            const float4 *s = reinterpret_cast<const float4 *>(R + hd.rs + 32 * rg);
            const float4 s0 = s[0], s1 = s[1];
            rr[0] = s0.x; rr[1] = s0.y; rr[2] = s0.z; rr[3] = s0.w;
            rr[4] = s1.x; rr[5] = s1.y; rr[6] = s1.z; rr[7] = s1.w;
        }
        if (A.cs16) {
            const uint4 s = *reinterpret_cast<const uint4 *>(R + hd.cs + 16 * cg);
            const uint32_t sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) { cc[2 * c] = f16v(sv[c]); cc[2 * c + 1] = f16v(sv[c] >> 16); }
        } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) cc[c] = 1.0f;
        }
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) { rr[c] = 0.0f; cc[c] = 1.0f; }
    }

    // decay + dequantize: A_ij
    float x[8][8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int w = rw.w[r];
        if (w == 16) {
            const uint32_t hv[4] = {raw[r].x, raw[r].y, raw[r].z, raw[r].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                x[r][2 * c] = aa[r] * f16v(hv[c]);
                x[r][2 * c + 1] = aa[r] * f16v(hv[c] >> 16);
            }
        } else {
            const float g = aa[r] * rr[r];
            const float nog = -(float)(1 << (w - 1)) * g;
            float u[8];
            codes_f(raw[r], w, u);
#pragma unroll
            for (int c = 0; c < 8; ++c) x[r][c] = fma_(u[c], g, nog) * cc[c];
        }
    }

    // w = (a.S) k : column partial sums over the thread's 8 rows
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        float s = x[0][c] * kk[0];
#pragma unroll
        for (int r = 1; r < 8; ++r) s = fma_(x[r][c], kk[r], s);
        sm.colp[rg][8 * cg + c] = s;
    }
    __syncthreads();
    if (t < DV) {
        float w = sm.colp[0][t];
#pragma unroll
        for (int g = 1; g < RG; ++g) w = w + sm.colp[g][t];
        sm.u[t] = beta * (vv - w);
    }
    __syncthreads();
    float uu[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) uu[c] = sm.u[8 * cg + c];

    // rank-1 write and o = S_new q partial sums
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) x[r][c] = fma_(kk[r], uu[c], x[r][c]);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        float s = x[0][c] * qq[0];
#pragma unroll
        for (int r = 1; r < 8; ++r) s = fma_(x[r][c], qq[r], s);
        sm.colp[rg][8 * cg + c] = s;
    }
    requant_store<DK, DV, W>(A, hd, R, rw, x, sm, t, rg, cg, true, unit);
}

template <int DK, int DV>
__global__ void __launch_bounds__(DK * DV / 64) k_step(Args A) {
    constexpr int CG = DV / 8;
    __shared__ Lds<DK, DV> sm;
    const size_t unit = blockIdx.x;
    const int b = (int)(unit / (size_t)A.H);
    const int h = (int)(unit - (size_t)b * A.H);
    const int t = threadIdx.x, rg = t / CG, cg = t - rg * CG;
    const int slot = A.slot_ids[b];
    if (slot < 0 || slot >= A.nslots) {
        // an invalid slot id touches no state; its output is NaN
        if (t < DV) A.o[unit * DV + t] = __builtin_nanf("");
        return;
    }
    const HeadDesc hd = A.heads[h];
    uint8_t *R = A.slots + (size_t)slot * A.slot_bytes + hd.off;

    float kk[8], qq[8], aa[8];
    load8(A.k, A.io_bf16, unit * DK + 8 * rg, kk);
    load8(A.q, A.io_bf16, unit * DK + 8 * rg, qq);
    if (A.gate_vec) {
        const float4 *p = reinterpret_cast<const float4 *>(A.a + unit * DK + 8 * rg);
        const float4 a0 = p[0], a1 = p[1];
        aa[0] = a0.x; aa[1] = a0.y; aa[2] = a0.z; aa[3] = a0.w;
        aa[4] = a1.x; aa[5] = a1.y; aa[6] = a1.z; aa[7] = a1.w;
    } else {
        const float a = A.a[unit];
#pragma unroll
        for (int r = 0; r < 8; ++r) aa[r] = a;
    }
    const float beta = A.beta[unit];
    const float vv = t < DV ? load1(A.v, A.io_bf16, unit * DV + t) : 0.0f;

    switch (hd.width) {
        case 4: step_tile<DK, DV, 4>(A, hd, R, sm, t, rg, cg, unit, kk, qq, aa, beta, vv); break;
        case 6: step_tile<DK, DV, 6>(A, hd, R, sm, t, rg, cg, unit, kk, qq, aa, beta, vv); break;
        case 8: step_tile<DK, DV, 8>(A, hd, R, sm, t, rg, cg, unit, kk, qq, aa, beta, vv); break;
        case 16: step_tile<DK, DV, 16>(A, hd, R, sm, t, rg, cg, unit, kk, qq, aa, beta, vv); break;
        default: step_tile<DK, DV, 0>(A, hd, R, sm, t, rg, cg, unit, kk, qq, aa, beta, vv); break;
    }
}

// ----------------------------------------------------------- pack / unpack

template <int DK, int DV, int W>
__device__ __forceinline__ void pack_tile(const Args &A, const HeadDesc &hd, uint8_t *R,
                                          Lds<DK, DV> &sm, int t, int rg, int cg, size_t unit) {
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
    requant_store<DK, DV, W>(A, hd, R, rw, x, sm, t, rg, cg, false, unit);
}

template <int DK, int DV>
__global__ void __launch_bounds__(DK * DV / 64) k_pack(Args A) {
    constexpr int CG = DV / 8;
    __shared__ Lds<DK, DV> sm;
    const size_t unit = blockIdx.x;
    const int b = (int)(unit / (size_t)A.H);
    const int h = (int)(unit - (size_t)b * A.H);
    const int t = threadIdx.x, rg = t / CG, cg = t - rg * CG;
    const int slot = A.slot_ids[b];
    if (slot < 0 || slot >= A.nslots) return;
    const HeadDesc hd = A.heads[h];
    uint8_t *R = A.slots + (size_t)slot * A.slot_bytes + hd.off;
    switch (hd.width) {
        case 4: pack_tile<DK, DV, 4>(A, hd, R, sm, t, rg, cg, unit); break;
        case 6: pack_tile<DK, DV, 6>(A, hd, R, sm, t, rg, cg, unit); break;
        case 8: pack_tile<DK, DV, 8>(A, hd, R, sm, t, rg, cg, unit); break;
        case 16: pack_tile<DK, DV, 16>(A, hd, R, sm, t, rg, cg, unit); break;
        default: pack_tile<DK, DV, 0>(A, hd, R, sm, t, rg, cg, unit); break;
    }
}

// Dequantized state: B_ij = RN(n_ij r_i c_j) (n r is exact), pivots as stored.
template <int DK, int DV>
__global__ void __launch_bounds__(DK * DV / 64) k_unpack(Args A) {
    constexpr int CG = DV / 8;
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
    const HeadDesc hd = A.heads[h];
    const uint8_t *R = A.slots + (size_t)slot * A.slot_bytes + hd.off;
    Rows rw;
    row_geometry<DV, 0>(A, hd, rg, rw);
    const bool quant = hd.nquant > 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int i = 8 * rg + r;
        const uint4 raw = load_piece(R + rw.ro[r], cg, rw.w[r]);
        float x[8];
        if (rw.w[r] == 16) {
            const uint32_t hv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) { x[2 * c] = f16v(hv[c]); x[2 * c + 1] = f16v(hv[c] >> 16); }
        } else {
            const float ri = !quant ? 0.0f
                             : A.rs16 ? f16v(reinterpret_cast<const uint16_t *>(R + hd.rs)[i])
                                      : reinterpret_cast<const float *>(R + hd.rs)[i];
            const float nor = -(float)(1 << (rw.w[r] - 1)) * ri;
            float u[8];
            codes_f(raw, rw.w[r], u);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float cj = (quant && A.cs16)
                                     ? f16v(reinterpret_cast<const uint16_t *>(R + hd.cs)[8 * cg + c])
                                     : 1.0f;
                x[c] = fma_(u[c], ri, nor) * cj;
            }
        }
        float4 *p = reinterpret_cast<float4 *>(dst + (size_t)i * DV + 8 * cg);
        p[0] = make_float4(x[0], x[1], x[2], x[3]);
        p[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
}

// ------------------------------------------------------------- pool init

__global__ void k_zero(uint4 *p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0, 0, 0, 0);
}

__global__ void k_gate_one(uint8_t *slots, uint64_t slot_bytes, int32_t nslots,
                           const HeadDesc *heads, int32_t H, int32_t dk) {
    const size_t n = (size_t)nslots * H * dk;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x) {
        const size_t s = i / ((size_t)H * dk);
        const int h = (int)((i / dk) % H);
        const int r = (int)(i % dk);
        reinterpret_cast<float *>(slots + s * slot_bytes + heads[h].off + heads[h].g)[r] = 1.0f;
    }
}

template <int DK, int DV>
hipError_t launch_dims(void (*k)(Args), const Args &a, hipStream_t s) {
    if (a.B == 0) return hipSuccess;
    hipLaunchKernelGGL(k, dim3((unsigned)((size_t)a.B * a.H)), dim3(DK * DV / 64), 0, s, a);
    return hipGetLastError();
}

}  // namespace

#define STQ_DISPATCH(KERNEL)                                                  \
    if (dk == 128 && dv == 128) return launch_dims<128, 128>(KERNEL<128, 128>, a, s); \
    if (dk == 64 && dv == 64) return launch_dims<64, 64>(KERNEL<64, 64>, a, s);       \
    if (dk == 128 && dv == 64) return launch_dims<128, 64>(KERNEL<128, 64>, a, s);    \
    if (dk == 64 && dv == 128) return launch_dims<64, 128>(KERNEL<64, 128>, a, s);    \
    return hipErrorInvalidValue;

hipError_t launch_step(const Args &a, int dk, int dv, hipStream_t s) { STQ_DISPATCH(k_step) }
hipError_t launch_pack(const Args &a, int dk, int dv, hipStream_t s) { STQ_DISPATCH(k_pack) }
hipError_t launch_unpack(const Args &a, int dk, int dv, hipStream_t s) { STQ_DISPATCH(k_unpack) }

hipError_t launch_pool_init(uint8_t *slots, uint64_t slot_bytes, int32_t nslots,
                            const HeadDesc *heads, int32_t H, int32_t dk, int32_t window,
                            hipStream_t s) {
    const size_t n16 = (size_t)nslots * slot_bytes / 16;
    if (n16 == 0) return hipSuccess;
    hipLaunchKernelGGL(k_zero, dim3(2048), dim3(256), 0, s, reinterpret_cast<uint4 *>(slots), n16);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || window <= 1) return e;
    hipLaunchKernelGGL(k_gate_one, dim3(1024), dim3(256), 0, s, slots, slot_bytes, nslots, heads, H, dk);
    return hipGetLastError();
}

}  // namespace stq
