// HIP kernels for gfx950: per-step decode, pack, unpack and pool init of the
// quantized recurrent state.  The arithmetic and the thread layout are
// described in stq_device.h.
#include "stq_device.h"

namespace stq {
using namespace dev;
namespace {

// ----------------------------------------------------------------- step

// The inputs of a 4-bit state that a workgroup fetches ahead of its compute:
// for thread t, the code piece of each of its 8 rows and its Inputs.
struct Pre4 {
    Inputs in;
    uint32_t raw[8];
};

template <int DK, int DV>
__device__ __forceinline__ void fetch4(const Args &A, const HeadDesc &hd, const uint8_t *R, size_t unit,
                                       int t, int rg, int cg, Pre4 &p) {
    const uint8_t *base = R + (uint32_t)(8 * rg * (DV / 2) + 4 * cg);
#pragma unroll
    for (int r = 0; r < 8; ++r) p.raw[r] = *reinterpret_cast<const uint32_t *>(base + r * (DV / 2));
    fetch_inputs<DK, DV>(A, hd, R, unit, t, p.in);
}

// One state.  PRE: a 4-bit state whose inputs were fetched into p (W == 4);
// otherwise the state's inputs are loaded here.
template <int DK, int DV, int W, bool PRE>
__device__ __forceinline__ void step_tile(const Args &A, const HeadDesc &hd, uint8_t *R, size_t unit,
                                          Lds<DK, DV> &sm, int t, int rg, int cg, const Pre4 &p) {
    static_assert(!PRE || W == 4, "prefetch is for 4-bit heads");
    const bool quant = has_quant<W>(hd);
    Rows rw;
    row_geometry<DV, W>(A, hd, rg, rw);
    uint4 raw[8];
    uint4 pv = make_uint4(0, 0, 0, 0);  // kW4P: the piece of the thread's first pivot row
    int pr = -1;                        //      and that row
    float x[8][8];                      // the thread's 8 x 8 block of the state
    if (W == 32) {
        // fp32 rows: the 8 values of each row piece straight into the block
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const float4 *p = reinterpret_cast<const float4 *>(R + row_o<DV, W>(rw, r) + 32 * cg);
            const float4 a0 = p[0], a1 = p[1];
            x[r][0] = a0.x; x[r][1] = a0.y; x[r][2] = a0.z; x[r][3] = a0.w;
            x[r][4] = a1.x; x[r][5] = a1.y; x[r][6] = a1.z; x[r][7] = a1.w;
        }
    } else if (PRE) {
#pragma unroll
        for (int r = 0; r < 8; ++r) raw[r] = make_uint4(p.raw[r], 0, 0, 0);
    } else if (W == kW4P) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            raw[r] = make_uint4(0, 0, 0, 0);
            if (row_w<W>(rw, r) != 16) {
                raw[r].x = *reinterpret_cast<const uint32_t *>(R + row_o<DV, W>(rw, r) + 4 * cg);
            } else if (pr < 0) {
                pv = load_piece(R + row_o<DV, W>(rw, r), cg, 16);
                pr = r;
            }
        }
    } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) raw[r] = load_piece(R + row_o<DV, W>(rw, r), cg, row_w<W>(rw, r));
    }

    // per key row and per value column constants, computed once per state
    Inputs own;
    if (!PRE) fetch_inputs<DK, DV>(A, hd, R, unit, t, own);
    const Inputs &in = PRE ? p.in : own;
    const float beta = in.beta;
    float vv = 0.0f;
    if (t < DK) {
        const int w = width_of<W>(A, hd, t);
        const float rl = dec_scale(in.r, A.rs16, t & 1);
        const float ri = (quant && w != 16) ? rl : 0.0f;
        const float g = in.a * ri;
        sm.g[t] = g;
        sm.g16[t] = g * 0.0625f;
        sm.nog[t] = w < 16 ? -(float)(1 << (w - 1)) * g : 0.0f;
        sm.af[t] = in.a;
        sm.kf[t] = dec_io(in.k, A.io_bf16, t & 1);
        sm.qf[t] = dec_io(in.q, A.io_bf16, t & 1);
    }
    if (t < DV) {
        const float c = dec_scale(in.c, 1, t & 1);
        sm.cf[t] = (quant && A.cs16) ? c : 1.0f;
        vv = dec_io(in.v, A.io_bf16, t & 1);
    }
    keep_inputs(in);
    __syncthreads();
    // decay + dequantize: A_ij, row by row, with the w = (a.S) k column
    // partial sums over the thread's 8 rows accumulated as the rows come in.
    // Vectors are read from LDS where they are used, so that none of them is
    // held across a barrier.
    {
        float kk[8], cc[8], s[8];
        lds_read8(&sm.kf[8 * rg], kk, 0);
        lds_read8(&sm.cf[8 * cg], cc, 0);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int i = 8 * rg + r;
            const int w = row_w<W>(rw, r);
            if (W == 32) {
                const float a = sm.af[i];
#pragma unroll
                for (int c = 0; c < 8; ++c) x[r][c] = a * x[r][c];
            } else if (w == 16) {
                const float a = sm.af[i];
                // kW4P: a second pivot row of the block is loaded here (rare)
                const uint4 pc = W != kW4P ? raw[r] : r == pr ? pv : load_piece(R + row_o<DV, W>(rw, r), cg, 16);
                const uint32_t hv[4] = {pc.x, pc.y, pc.z, pc.w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    x[r][2 * c] = a * f16v(hv[c]);
                    x[r][2 * c + 1] = a * f16v(hv[c] >> 16);
                }
            } else {
                dequant_row(raw[r], W == kW4P ? 4 : w, sm.g[i], sm.g16[i], sm.nog[i], x[r]);
#pragma unroll
                for (int c = 0; c < 8; ++c) x[r][c] = x[r][c] * cc[c];
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) s[c] = r == 0 ? x[0][c] * kk[0] : fma_(x[r][c], kk[r], s[c]);
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) sm.colp[c][t] = s[c];
    }
    __syncthreads();
    if (t < DV) sm.u[t] = beta * (vv - col_sum<DK, DV>(sm, t));
    __syncthreads();

    // rank-1 write, then o = S_new q partial sums
    {
        float kk[8], uu[8];
        lds_read8(&sm.kf[8 * rg], kk, 0);
        lds_read8(&sm.u[8 * cg], uu, 0);
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int c = 0; c < 8; ++c) x[r][c] = fma_(kk[r], uu[c], x[r][c]);
    }
    {
        float qq[8];
        lds_read8(&sm.qf[8 * rg], qq, 0);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float s = x[0][c] * qq[0];
#pragma unroll
            for (int r = 1; r < 8; ++r) s = fma_(x[r][c], qq[r], s);
            sm.colp[c][t] = s;
        }
    }
    requant_store<DK, DV, W>(A, hd, R, rw, x, sm, t, rg, cg, true, unit);
}


// Workgroup g steps the states of head group g % ngroups of request
// g / ngroups.  A group is one head, or two 4-bit heads: then the second
// state's inputs are fetched before the first is computed, so their latency
// is hidden behind that compute (workgroup barriers wait only for LDS
// traffic).  MIX: 0 if every head has one row width, 1 if the other heads
// are all 4-bit rows with FP16 pivot rows (kW4P), 2 if some head mixes other
// widths; only the per-row paths a layout needs are compiled, which saves
// registers.
template <int DK, int DV, int MIX>
__global__ void __launch_bounds__(DK * DV / 64) k_step(Args A) {
    constexpr int CG = DV / 8;
    __shared__ Lds<DK, DV> sm;
    // ngroups == 0: every head alone (small batches keep more workgroups)
    const int ng = A.ngroups ? A.ngroups : A.H;
    const int b = (int)(blockIdx.x / (uint32_t)ng);
    const int gi = (int)(blockIdx.x - (uint32_t)b * ng);
    const uint32_t grp = A.ngroups ? A.groups[gi] : ((uint32_t)gi | 0xffff0000u);
    const int h1 = (int)(grp & 0xffffu), h2 = (int)(grp >> 16);
    const int t = threadIdx.x, rg = t / CG, cg = t - rg * CG;
    const size_t u1 = (size_t)b * A.H + h1;
    const int slot = A.slot_ids[b];
    if (slot < 0 || slot >= A.nslots) {
        // an invalid slot id touches no state; its outputs are NaN
        if (t < DV) {
            A.o[u1 * DV + t] = __builtin_nanf("");
            if (h2 != 0xffff) A.o[((size_t)b * A.H + h2) * DV + t] = __builtin_nanf("");
        }
        return;
    }
    uint8_t *S = A.slots + (size_t)slot * A.slot_bytes;
    const HeadDesc &hd1 = A.heads[h1];
    if (h2 != 0xffff) {
        const HeadDesc &hd2 = A.heads[h2];
        const size_t u2 = (size_t)b * A.H + h2;
        Pre4 p1, p2;
        fetch4<DK, DV>(A, hd1, S + hd1.off, u1, t, rg, cg, p1);
        __builtin_amdgcn_sched_barrier(0);  // keep the first state's loads ahead
        fetch4<DK, DV>(A, hd2, S + hd2.off, u2, t, rg, cg, p2);
        step_tile<DK, DV, 4, true>(A, hd1, S + hd1.off, u1, sm, t, rg, cg, p1);
        step_tile<DK, DV, 4, true>(A, hd2, S + hd2.off, u2, sm, t, rg, cg, p2);
        return;
    }
    uint8_t *R = S + hd1.off;
    Pre4 none;
    switch (head_width(hd1)) {
        case 4: step_tile<DK, DV, 4, false>(A, hd1, R, u1, sm, t, rg, cg, none); break;
        case 6: step_tile<DK, DV, 6, false>(A, hd1, R, u1, sm, t, rg, cg, none); break;
        case 8: step_tile<DK, DV, 8, false>(A, hd1, R, u1, sm, t, rg, cg, none); break;
        case 16: step_tile<DK, DV, 16, false>(A, hd1, R, u1, sm, t, rg, cg, none); break;
        case 32: step_tile<DK, DV, 32, false>(A, hd1, R, u1, sm, t, rg, cg, none); break;
        case kW4P:
            if (MIX >= 1) step_tile<DK, DV, kW4P, false>(A, hd1, R, u1, sm, t, rg, cg, none);
            break;
        default:
            if (MIX == 2) step_tile<DK, DV, 0, false>(A, hd1, R, u1, sm, t, rg, cg, none);
            break;
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
    switch (head_width(hd)) {
        case 4: pack_tile<DK, DV, 4>(A, hd, R, sm, t, rg, cg, unit); break;
        case 6: pack_tile<DK, DV, 6>(A, hd, R, sm, t, rg, cg, unit); break;
        case 8: pack_tile<DK, DV, 8>(A, hd, R, sm, t, rg, cg, unit); break;
        case 16: pack_tile<DK, DV, 16>(A, hd, R, sm, t, rg, cg, unit); break;
        case 32: pack_tile<DK, DV, 32>(A, hd, R, sm, t, rg, cg, unit); break;
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
    const bool quant = head_nquant(hd) > 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int i = 8 * rg + r;
        float x[8];
        if (rw.w[r] == 32) {
            const float4 *p = reinterpret_cast<const float4 *>(R + rw.ro[r] + 32 * cg);
            const float4 a0 = p[0], a1 = p[1];
            x[0] = a0.x; x[1] = a0.y; x[2] = a0.z; x[3] = a0.w;
            x[4] = a1.x; x[5] = a1.y; x[6] = a1.z; x[7] = a1.w;
        } else if (rw.w[r] == 16) {
            const uint4 raw = load_piece(R + rw.ro[r], cg, 16);
            const uint32_t hv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int c = 0; c < 4; ++c) { x[2 * c] = f16v(hv[c]); x[2 * c + 1] = f16v(hv[c] >> 16); }
        } else {
            const uint4 raw = load_piece(R + rw.ro[r], cg, rw.w[r]);
            const float ri = !quant ? 0.0f
                             : A.rs16 ? f16v(reinterpret_cast<const uint16_t *>(R + hd.rs)[i])
                                      : reinterpret_cast<const float *>(R + hd.rs)[i];
            dequant_row(raw, rw.w[r], ri, ri * 0.0625f, -(float)(1 << (rw.w[r] - 1)) * ri, x);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float cj = (quant && A.cs16)
                                     ? f16v(reinterpret_cast<const uint16_t *>(R + hd.cs)[8 * cg + c])
                                     : 1.0f;
                x[c] = x[c] * cj;
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

// Heads are paired only when the batch leaves enough workgroups to fill the
// chip several times over.
constexpr size_t kPairMinStates = 8192;

template <int DK, int DV, int MIX>
hipError_t launch_step_dims(Args a, hipStream_t s) {
    if (a.B == 0) return hipSuccess;
    if ((size_t)a.B * a.H < kPairMinStates) a.ngroups = 0;
    const size_t per_request = a.ngroups ? (size_t)a.ngroups : (size_t)a.H;
    void (*k)(Args) = k_step<DK, DV, MIX>;
    hipLaunchKernelGGL(k, dim3((unsigned)((size_t)a.B * per_request)), dim3(DK * DV / 64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_step(const Args &a, int dk, int dv, int mix, hipStream_t s) {
#define STQ_STEP(DK_, DV_)                                                                      \
    if (dk == DK_ && dv == DV_)                                                                 \
        return mix == 2 ? launch_step_dims<DK_, DV_, 2>(a, s)                                  \
                        : mix == 1 ? launch_step_dims<DK_, DV_, 1>(a, s) : launch_step_dims<DK_, DV_, 0>(a, s);
    STQ_STEP(128, 128)
    STQ_STEP(64, 64)
    STQ_STEP(128, 64)
    STQ_STEP(64, 128)
#undef STQ_STEP
    return hipErrorInvalidValue;
}
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
