/*
 * stq.h — C ABI of the MI355X (gfx950) quantized-recurrent-state decode library.
 *
 * The library steps the recurrent state of a gated delta-rule linear-attention
 * layer for a batch of requests, one token per call.  Each request's state
 * lives in a caller-owned device pool, quantized in the STEPQuant style: a bit
 * width per unit (a whole head for GDN, one key row for KDA) from {4,6,8},
 * FP16 pivot units, and a row scale and a column scale per state refitted every
 * step (STEPQuant essay: temporal-axis, spatial-axis and experiment-design
 * paragraphs).  A windowed mode keeps the low-bit base fixed for W tokens with
 * fp32 rank-1 deltas and K fp32 compensation entries (LeapQuant article,
 * "研究の概要").
 *
 * Conventions for every call:
 *  - Every call returns stq_status; nothing throws across the ABI.
 *  - Arguments are validated on the host before anything is launched; a
 *    rejected call writes nothing, on the host or the device.
 *  - No call synchronizes the device; work is queued on `stream` (a
 *    hipStream_t; NULL is the default stream).  Launch failures return
 *    STQ_ERR_DEVICE with the HIP error text in stq_last_error().  (A library
 *    built with STQ_DEBUG_VALIDATE copies slot ids back to the host to check
 *    them, which synchronizes; see stq_check_slot_ids.)
 *  - Device memory is always the caller's; the library never allocates it.
 *    Device pointers must be 16-byte aligned (slot ids: 4-byte).
 *  - A pool must not be used by two calls that overlap in time (e.g. on two
 *    streams).  Layouts are immutable once built and may be shared.
 *
 * State orientation: M = S^T, d_k x d_v, key-row-major; row i is key channel
 * i, column j is value channel j.  Arithmetic (every rounding, the summation
 * order) and the storage format are fixed so that results are reproducible
 * bit for bit; they are stated where the library's sources define them.
 */
#ifndef STQ_H
#define STQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    STQ_OK = 0,
    STQ_ERR_INVALID = 1,      /* bad argument (NULL, out of range, inconsistent) */
    STQ_ERR_UNSUPPORTED = 2,  /* valid but not supported (e.g. d not 64/128) */
    STQ_ERR_TOO_SMALL = 3,    /* caller buffer too small */
    STQ_ERR_ALIGN = 4,        /* misaligned device pointer */
    STQ_ERR_DEVICE = 5        /* HIP launch / runtime error */
} stq_status;

enum { STQ_UNIT_HEAD = 0, STQ_UNIT_KEYROW = 1 };      /* quantization unit */
enum { STQ_GATE_SCALAR = 0, STQ_GATE_KEYVEC = 1 };    /* gate a: [B,H] or [B,H,d_k] */
enum { STQ_NONE = 0, STQ_F32 = 1, STQ_F16 = 2, STQ_BF16 = 3 };
enum { STQ_FIT_STEP = 0, STQ_FIT_LAGGED = 1 };       /* where the scales are fitted */

/* Layer configuration.  unit_bits is read during stq_pack_layout only. */
typedef struct {
    int32_t H;               /* heads, >= 1 */
    int32_t d_k, d_v;        /* 64 or 128 each */
    int32_t unit;            /* STQ_UNIT_HEAD (GDN) | STQ_UNIT_KEYROW (KDA) */
    int32_t gate;            /* STQ_GATE_SCALAR | STQ_GATE_KEYVEC */
    int32_t row_scale;       /* STQ_F16 | STQ_F32 */
    int32_t col_scale;       /* STQ_F16 | STQ_NONE */
    int32_t io_dtype;        /* q, k, v: STQ_BF16 | STQ_F32 (o is always fp32) */
    int32_t window;          /* 1: requantize every step; 2..16: windowed */
    int32_t comps;           /* windowed: K fp32 compensation entries, 0..1024 */
    int32_t scale_fit;       /* STQ_FIT_STEP: scales refitted inside each step;
                                STQ_FIT_LAGGED: the step writes with scales fitted
                                to the previous state, stq_fit_scales fits the next
                                (every-step mode, heads of one width each) */
    const uint8_t *unit_bits;/* host; H (per head) or H*d_k (per key row) widths
                                in {4,6,8,16,32}; 16 = FP16 pivot unit; 32 = fp32
                                (unquantized) unit: window 1 only, whole heads */
    const float *row_impact; /* host, NULL or [H*d_k] row-impact scores >= 0 (STEPQuant
                                essay, spatial-axis paragraph), fixed offline: the
                                column scales are fitted to max_i w_i |M_ij| with
                                w_i = sqrt(score_i / the head's largest score) (1 when
                                a head's scores are all 0); every-step mode with
                                STQ_FIT_STEP only */
} stq_config;

typedef struct stq_layout stq_layout;   /* opaque, host-owned by the library */

/* Static text of a status code. */
const char *stq_status_string(stq_status s);

/* Detail of the last failing call on this thread ("" if none). */
const char *stq_last_error(void);

/*
 * Validate a configuration and compute the slot layout (STEPQuant essay,
 * experiment-design paragraph: widths and pivots are fixed offline, scales are
 * refitted online).  On success *out owns a new layout; free it with
 * stq_layout_free.  Errors: STQ_ERR_INVALID (NULL, H < 1, widths not in
 * {4,6,8,16,32}, bad enums, comps without window, comps > quantized entries),
 * STQ_ERR_UNSUPPORTED (d_k or d_v not 64/128, window > 16, fp32 units in the
 * windowed mode or on part of a head's key rows, lagged scales with the
 * windowed mode or with key rows of different widths in one head, row-impact
 * scores with the windowed mode or lagged scales; a negative or non-finite
 * score is STQ_ERR_INVALID).
 */
stq_status stq_pack_layout(const stq_config *cfg, stq_layout **out);

/* Bytes of one slot (one request, all heads of one layer) and of the pool's
 * table header.  Either output may be NULL. */
stq_status stq_layout_query(const stq_layout *layout, size_t *slot_bytes, size_t *header_bytes);

/* Byte offset and size of head h's region inside a slot. */
stq_status stq_layout_head(const stq_layout *layout, int32_t h, size_t *offset, size_t *bytes);

void stq_layout_free(stq_layout *layout);

/* A pool view over caller memory: [table header][slot 0][slot 1]... */
typedef struct {
    void *base;                 /* device pointer to the caller's buffer */
    size_t bytes;               /* bytes required / used */
    int32_t slots;              /* number of slots */
    const stq_layout *layout;   /* layout the pool was carved for (not owned) */
} stq_pool;

/*
 * Reserve `slots` request slots in caller device memory (STEPQuant essay,
 * opening paragraphs: the serving system keeps a reserved per-request state
 * pool).  dev_base == NULL: only sets out->bytes to the required size.
 * Otherwise dev_bytes must be >= that size; the table header is uploaded and
 * every slot is set to the empty state (zero state, cumulative gates 1, no
 * deltas), asynchronously on `stream`.  Slot s starts at
 * base + header_bytes + s * slot_bytes.  Windowed layouts keep an 8-byte
 * window-end flag at the end of the header, written by stq_decode_step: the
 * header of such a pool is not read-only while it is stepped.
 */
stq_status stq_alloc_pool(const stq_layout *layout, int32_t slots, void *dev_base,
                          size_t dev_bytes, void *stream, stq_pool *out);

/*
 * One decode step for B requests (gated delta rule, STEPQuant essay background
 * paragraph; LeapQuant "研究の概要" for the windowed mode):
 *   d_slot_ids [B] int32   slot of each request, distinct, in [0, slots)
 *   d_q, d_k   [B,H,d_k]   io_dtype
 *   d_v        [B,H,d_v]   io_dtype
 *   d_a        [B,H] fp32 (scalar gate) or [B,H,d_k] fp32 (key-vector gate)
 *   d_beta     [B,H] fp32  write strength
 *   d_o        [B,H,d_v] fp32 output o = S_new q
 * Per state: dequantize, decay, w = (a*S)k, u = beta(v - w), S += u k^T,
 * o = S q, refit column then row scales, requantize and write back (windowed:
 * append the delta; requantize at the window end).  B may be 0 (no-op).
 * The call allocates nothing and does not synchronize, so it may be captured
 * in a HIP graph; a replayed windowed call reuses its captured token, which
 * costs the window-end kernel a per-state check on every replay but changes
 * no result.
 */
stq_status stq_decode_step(const stq_pool *pool, int32_t B, const int32_t *d_slot_ids,
                           const void *d_q, const void *d_k, const void *d_v,
                           const float *d_a, const float *d_beta, float *d_o, void *stream);

/*
 * Current state of B slots as fp32 [B,H,d_k,d_v] (key-row-major): the
 * dequantized codes (n * r * c, FP16 pivots as stored; windowed: the base with
 * its compensation entries, materialized with the stored deltas and gate).
 * This is the "unpack" stage of the fused decode kernel (STEPQuant essay,
 * experiment-design paragraph: the state is unpacked, updated and written out
 * in one kernel) offered on its own; for the windowed mode it is the
 * materialization of the fixed low-bit base, the fp32 window updates and the
 * compensation entries (LeapQuant article, "研究の概要").
 *   d_slot_ids [B] int32  device, distinct, in [0, slots); an id out of range
 *                         gives NaN for that request's states
 *   d_state    [B,H,d_k,d_v] fp32 device output, 16-byte aligned
 * Errors: STQ_ERR_INVALID (NULL pool/ids/state, B < 0 or B > slots),
 * STQ_ERR_ALIGN, STQ_ERR_DEVICE; nothing is written then.
 */
stq_status stq_unpack(const stq_pool *pool, int32_t B, const int32_t *d_slot_ids,
                      float *d_state, void *stream);

/*
 * Quantize fp32 states [B,H,d_k,d_v] into B slots (column then row absmax
 * scales, codes, FP16 pivots; windowed: top-K compensation entries, gate 1,
 * no deltas).  Used to seed initial states and to inspect requantization.
 * This is the "write out" stage of the fused decode kernel with its scale
 * fitting and compressed store (STEPQuant essay, experiment-design paragraph:
 * the dual-axis scales are refitted to the state being stored); for the
 * windowed mode it is the requantization at a window end, with the largest
 * entries kept at high precision (LeapQuant article, "研究の概要").
 *   d_slot_ids [B] int32  device, distinct, in [0, slots); an id out of range
 *                         is skipped (nothing written for that request)
 *   d_state    [B,H,d_k,d_v] fp32 device input, 16-byte aligned, not modified
 * Errors: as stq_unpack.
 */
stq_status stq_pack(const stq_pool *pool, int32_t B, const int32_t *d_slot_ids,
                    const float *d_state, void *stream);

/*
 * Lagged scales (STQ_FIT_LAGGED layouts): fit the next scales of B slots from
 * the statistics their last stq_decode_step recorded (STEPQuant essay,
 * experiment-design paragraph: the scale fitting runs on a separate stream so
 * that it does not block the decode path, while unpack, update and write-out
 * are one fused kernel).  Per head with quantized rows: next column scale
 * c~_j = H(column absmax), next row scale r~_i = smallest fp16 (fp32 row
 * scales: the fp32) not below (row absmax in that column scale) / qmax_i.
 * Meant for a second stream: the caller orders it after the decode step it
 * follows (an event) and before the next decode step of the same slots.
 * A slot that was never stepped (or was just packed) has no statistics; its
 * next step refits in the step.
 *   d_slot_ids [B] int32 device, distinct, in [0, slots); out-of-range ids are
 *                       skipped
 * Errors: STQ_ERR_INVALID (NULL pool/ids, B < 0 or B > slots, a layout
 * without lagged scales), STQ_ERR_ALIGN, STQ_ERR_DEVICE.
 */
stq_status stq_fit_scales(const stq_pool *pool, int32_t B, const int32_t *d_slot_ids, void *stream);

/*
 * Host check of a batch's slot ids: every id in [0, pool->slots) and no id
 * twice.  Two requests of one call on the same slot would make two workgroups
 * read-modify-write one state with no ordering between them, so the calls
 * require distinct ids (the serving pool keeps one reserved slot per live
 * request: STEPQuant essay, opening paragraphs).  The release library does
 * not copy device ids back to check them on every call (that would
 * synchronize the stream); a library built with STQ_DEBUG_VALIDATE does, and
 * then rejects a bad batch in stq_decode_step, stq_unpack and stq_pack before
 * anything is launched.
 *   h_slot_ids [B] int32 host
 * Returns STQ_OK, or STQ_ERR_INVALID naming the first bad position.
 */
stq_status stq_check_slot_ids(const stq_pool *pool, int32_t B, const int32_t *h_slot_ids);

/*
 * Lifetime-aware bit allocation (host only; STEPQuant essay, temporal-axis
 * paragraphs and the Proposition 1 discussion: an error that the update does
 * not remove fades only by the gate, so long-lived units get more bits within
 * a fixed average, and the riskiest few stay FP16 pivots).  Fills unit_bits
 * for stq_config.unit_bits from per-unit calibration statistics:
 *   n_units      units of one layer: H (per head) or H*d_k (per key row)
 *   gate_mean    [n_units] host, mean gate of the unit, in [0, 1]
 *   state_msq    [n_units] host, mean squared state entry of the unit, >= 0
 *   avg_bits     mean width over the non-pivot units, in [4, 8]
 *   n_pivots     units kept as FP16 pivots (width 16), in [0, n_units]
 *   unit_bits    [n_units] host output: 4, 6, 8 or 16
 * Weight s = state_msq / (1 - min(gate_mean, 1 - 2^-20)); the n_pivots largest
 * weights become pivots; the others start at 4 and, while 2 more bits fit in
 * floor(avg_bits * (n_units - n_pivots)), the unit with the largest
 * s * (4^-b - 4^-(b+2)) gains 2 bits (ties: lower index), up to 8.  Double
 * arithmetic; deterministic.  Errors: STQ_ERR_INVALID (NULL, n_units < 1,
 * avg_bits or n_pivots out of range, a statistic out of range or not finite);
 * nothing is written then.
 */
stq_status stq_allocate_bits(int32_t n_units, const float *gate_mean, const float *state_msq,
                             double avg_bits, int32_t n_pivots, uint8_t *unit_bits);

#ifdef __cplusplus
}
#endif

#endif /* STQ_H */
