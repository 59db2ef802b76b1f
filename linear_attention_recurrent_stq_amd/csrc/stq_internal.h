// Internal definitions shared by the host side (stq_host.cpp) and the gfx950
// kernels (stq_kernels.hip).  Not part of the ABI.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

namespace stq {

// Per-head entry of the device layout table (in the pool header).  Offsets
// are in bytes from the start of the head's region inside a slot.
struct HeadDesc {
    uint32_t off;      // region offset inside the slot
    uint32_t bytes;    // region size
    uint32_t rs;       // row scales (valid if nquant > 0)
    uint32_t cs;       // column scales (valid if nquant > 0 and column scales on)
    // The windowed sections and the lagged-scale sections never share a
    // layout, so they share these six offsets.
    union {
        struct {
            uint32_t wn;       // windowed: delta count (int32)
            uint32_t g;        // windowed: cumulative gate [d_k] fp32
            uint32_t cidx;     // windowed: compensation index [K] uint16
            uint32_t cval;     // windowed: compensation value [K] fp32
            uint32_t du;       // windowed: delta values [W][d_v] fp32
            uint32_t dkap;     // windowed: delta keys [W][d_k] fp32
        };
        struct {
            uint32_t nrs;      // lagged: next row scales [d_k] (as the row scales)
            uint32_t ncs;      // lagged: next column scales [d_v] fp16 (if column scales)
            uint32_t srs;      // lagged: row statistics [d_k] fp32
            uint32_t scs;      // lagged: column statistics [d_v] fp32 (if column scales)
            uint32_t spare0, spare1;
        };
    };
    uint32_t rows;     // first entry of this head in the row table
    union {
        struct {
            uint16_t width;    // width shared by every row (4/6/8/16); kW4P: 4-bit rows and
                               // FP16 pivot rows; 0: rows of other differing widths
            uint16_t nquant;   // number of quantized (non-pivot) rows
        };
        uint32_t wq;           // both, as one dword (width | nquant << 16)
    };
    uint32_t pmask[4]; // kW4P heads: bit i % 32 of word i / 32 set if key row i is an
                       // FP16 pivot row (the row offsets follow from it); else 0
};
static_assert(sizeof(HeadDesc) == 64, "HeadDesc is 64 bytes");

// HeadDesc::width of a head whose rows are 4-bit or FP16 pivots (and not all
// the same): such heads are stepped by a path holding one dword per row.
constexpr uint16_t kW4P = 20;

// Row table entry: (byte offset of the row inside the head region) << 6 | width
// (widths 4, 6, 8, 16 and 32 need six bits; offsets stay below 2^26).
__host__ __device__ inline uint32_t row_entry(uint32_t off, uint32_t width) { return (off << 6) | width; }
__host__ __device__ inline uint32_t row_off(uint32_t e) { return e >> 6; }
__host__ __device__ inline uint32_t row_width(uint32_t e) { return e & 63u; }

// Kernel arguments (passed by value).
struct Args {
    uint8_t *slots;              // first slot (pool base + header bytes)
    const HeadDesc *heads;       // [H]
    const uint32_t *rows;        // [H * d_k]
    uint64_t slot_bytes;
    const int32_t *slot_ids;     // [B]
    const void *q, *k, *v;       // [B,H,d] io dtype
    const float *a;              // [B,H] or [B,H,d_k]
    const float *beta;           // [B,H]
    float *o;                    // [B,H,d_v]
    float *state;                // pack / unpack: [B,H,d_k,d_v]
    int32_t B, H, nslots;
    int32_t io_bf16, gate_vec, rs16, cs16;
    int32_t window, comps;
    int32_t lagged;              // STQ_FIT_LAGGED layout
    const uint32_t *groups;      // step kernel: [ngroups] head groups, h1 | h2 << 16
    int32_t ngroups;             //   (h2 = 0xffff: a group of one head)
    const float *omega;          // row-impact weights [H * d_k] (nullptr: none)
    // Windowed layouts: a flag in the pool header that the in-window step sets
    // to `token` (unique to the call) when one of its states fills its window,
    // so that the window-end kernel can tell at once that none did.
    uint64_t *end_flag;
    uint64_t token;
};

// Launchers (stq_kernels.hip).  Return the launch's hipError_t.  `mixed`: some
// head of the layout has rows of different widths; `mix`: 0 none, 1 only
// kW4P heads, 2 other mixed heads.
hipError_t launch_step(const Args &a, int dk, int dv, int mix, hipStream_t s);
// Lagged scales: the step (heads of one width) and the fit of the next scales.
hipError_t launch_step_lagged(const Args &a, int dk, int dv, hipStream_t s);
hipError_t launch_fit(const Args &a, int dk, int dv, hipStream_t s);
hipError_t launch_pack(const Args &a, int dk, int dv, hipStream_t s);
hipError_t launch_unpack(const Args &a, int dk, int dv, hipStream_t s);
// Windowed layouts (window > 1): stq_window.hip.
hipError_t launch_step_win(const Args &a, int dk, int dv, bool mixed, hipStream_t s);
hipError_t launch_pack_win(const Args &a, int dk, int dv, bool mixed, hipStream_t s);
hipError_t launch_unpack_win(const Args &a, int dk, int dv, hipStream_t s);
hipError_t launch_pool_init(uint8_t *slots, uint64_t slot_bytes, int32_t nslots,
                            const HeadDesc *heads, int32_t H, int32_t dk, int32_t window,
                            hipStream_t s);

}  // namespace stq
