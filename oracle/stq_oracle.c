/*
 * Oracle for the quantized-recurrent-state decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header or table with the HIP
 * library.
 *
 * What it computes (plain, slow, single-threaded, fp32 with every rounding
 * written out so that an independent implementation can match it bit for bit):
 *
 *  - The gated delta-rule decode step of one (request, head) state
 *    (STEPQuant essay, background paragraph on linear attention and the gated
 *    delta rule; LeapQuant article, "研究の概要"):
 *        S <- a*S + beta*(v - a*S*k) k^T ,   o = S q
 *    kept as M = S^T (d_k x d_v, key-row-major), gate a per key row (KDA) or
 *    one scalar per head (GDN).
 *  - Quantized storage in the STEPQuant style (essay, temporal-axis and
 *    spatial-axis paragraphs): a bit width per unit (a whole head for GDN, one
 *    key row for KDA) from {4,6,8}, FP16 pivot units (width 16), fp32 units
 *    (width 32: the unquantized state the pages compare against), and a row
 *    scale and a column scale per state (dual-axis fitting), refitted at every
 *    step from absolute maxima (essay, experiment-design paragraph: the
 *    dual-axis scales are recomputed each decode step).
 *  - The windowed variant (LeapQuant article, "研究の概要", first and second
 *    device): the low-bit base is fixed inside a window of W tokens, updates
 *    are kept as fp32 rank-1 deltas, and only at the window end is the state
 *    materialized, its K largest-magnitude entries kept as fp32 compensation
 *    values and the rest requantized.
 *
 * The pages give no formulas, no rounding and no summation order.  The
 * readings used here (one per open point) are:
 *   RN(x)      fp32 round-to-nearest-even of the exact value.
 *   fma        one rounding of the exact a*b+c.
 *   H(x)       fp16 round-to-nearest-even after clamping to +-65504.
 *   Hup(x)     smallest fp16 >= x (x >= 0), at most 65504.
 *   csum(x,y)  sum_i x_i*y_i over i = 0..d_k-1: blocks of 8 consecutive i,
 *              each s = RN(x0*y0) then s = fma(x_t, y_t, s); block sums are
 *              then added left to right with RN.
 *   codes      offset binary: stored u = n + 2^(b-1), n in [-qmax, qmax],
 *              qmax = 2^(b-1)-1; row i is a little-endian LSB-first bit
 *              stream, code j at bits [j*b, (j+1)*b).
 *
 * Per-step mode (window == 1), one state.  The stored state is the product
 * diag(r) N diag(c) of the dual-axis fit; the step keeps it in that factored
 * form: the row factor (with the gate) scales the codes, and the column
 * factor s_j multiplies each column once, on the value side (w, o, u),
 * instead of every entry.  The working state M''_ij = M_ij / s_j is the
 * state in units of the stored column scale.
 *   column factor  s_j = c_j if column scales are on and c_j > 0, else 1;
 *                  is_j = RN(1/s_j)
 *   decay+dequant  g_i = RN(a_i*r_i);  A_ij = RN(n_ij*g_i)
 *                  pivot row: A_ij = RN(RN(a_i*h_ij)*is_j);
 *                  fp32 row: A_ij = RN(a_i*m_ij) (fp32 heads have s = 1)
 *   read           w_j = RN(s_j*csum(A_.j, k))
 *   delta          u_j = RN(beta*RN(v_j - w_j));  u'_j = RN(u_j*is_j)
 *   write          M''_ij = fma(k_i, u'_j, A_ij)
 *   output         o_j = RN(s_j*csum(M''_.j, q))
 *   column scale   C_j = max over non-pivot rows |M''_ij|; c'_j = H(RN(C_j*s_j));
 *                  f_j = c'_j > 0 ? RN(s_j/c'_j) : 0;  Z_ij = RN(M''_ij*f_j)
 *                  (no column scale: Z = M'')
 *   row scale      R_i = max_j |Z_ij|;  r'_i = Hup(RN(R_i/qmax_i))  (fp32 row
 *                  scale: r'_i = RN(R_i/qmax_i));  ir_i = RN(1/r'_i), or 0 when
 *                  r'_i = 0 or 1/r'_i overflows.  Rounding the step up means
 *                  |Z_ij*ir_i| < qmax + 1/2, so the clamp below only acts when
 *                  the step saturated at 65504.
 *   codes          n'_ij = clamp(rne(Z_ij*ir_i exactly), -qmax_i, qmax_i)
 *                  pivot row: h'_ij = H(RN(M''_ij*s_j)); fp32 row: m'_ij = M''_ij
 *                  (pivot and fp32 rows are left out of both scale maxima)
 * Requantizing an fp32 state M directly (pack, window end) is the same with
 * s = 1: c'_j = H(C_j), f_j = RN(1/c'_j).
 *
 * Row-impact weighting (row_impact given; STEPQuant essay, spatial-axis
 * paragraph: each key row's contribution to the output error is scored, and
 * experiment-design paragraph: the column scale penalizes reconstruction
 * error on high-impact rows, large-value rows get a wide range and important
 * rows a finer resolution).  With impact iota_i >= 0 per key row of a head,
 * w_i = RN(sqrt(iota_i / max_k iota_k)) (computed in double; 1 when the
 * head's impacts are all 0), the column maximum becomes
 * C_j = max over quantized rows RN(w_i |M''_ij|); the row scale is fitted as
 * above, to the row's current magnitude in those column units.
 *
 * Lagged scales (scale_fit == 1; every-step mode).  The scale fit runs apart
 * from the decode step (STEPQuant essay, experiment-design paragraph: scale
 * fitting and the compressed store run on a separate stream, while unpack,
 * update and write-out are one fused kernel).  A head keeps, besides the
 * scales r, c its codes are in, the next scales rn, cn to write with, and the
 * statistics of its last step: SC_j (column absmax) and SR_i (row absmax in
 * the column scale it was written with).
 *   step, when some quantized row has rn_i > 0: the update as above, then
 *     the statistics are the refit the every-step mode would make of this
 *     state: SC_j = RN(max over quantized rows |M''_ij| * s_j),
 *     SR_i = max_j |RN(M''_ij*RN(s_j/H(SC_j)))| (0 factor when H(SC_j) = 0);
 *     the codes are written with the next scales:
 *     f_j = cn_j > 0 ? RN(s_j/cn_j) : 0;  Z_ij = RN(M''_ij*f_j) (no column
 *     scale: Z = M'', SR_i = max_j |M''_ij|);  irn_i = RN(1/rn_i) (0 when
 *     rn_i = 0 or it overflows);  n'_ij = clamp(rne(Z_ij*irn_i exactly),
 *     -qmax_i, qmax_i) -- the scales were fitted to the previous state, so
 *     entries can clip;  pivot rows as above;  r = rn, c = cn.
 *   step, when no quantized row has rn_i > 0 (a fresh or zero state): the
 *     every-step refit above, with SC_j = RN(max |M''_ij| * s_j) and
 *     SR_i = max_j |Z_ij| of that refit.
 *   fit (a call of its own): rn_i = Hup(RN(SR_i/qmax_i)) (fp32 row scales:
 *     RN(SR_i/qmax_i)), 0 on pivot rows;  cn_j = H(SC_j).
 *
 * Windowed mode (window W > 1), base B_ij = RN(n_ij*r_i*c_j) (pivot: h_ij;
 * compensation positions: their fp32 value), cumulative gate g (1 at a
 * window start), deltas (u_m, kap_m), m = 1..n:
 *   kap_m,i = RN(kap_m,i*a_i);  g_i = RN(g_i*a_i)
 *   w_j = csum(Bq_.j, RN(g*k)), Bq = B without its compensation entries;
 *         then each compensation entry (i, j, val) of column j, in index
 *         order: w_j = fma(val, RN(g_i*k_i), w_j)  (a compensation entry is a
 *         token with a one-hot key on the ordinary update path);
 *         then w_j = fma(u_m,j, csum(kap_m, k), w_j), m = 1..n
 *   u_j = RN(beta*RN(v_j - w_j));  append (u, kap = k)
 *   o_j: the same with q in place of k, over m = 1..n+1
 *   at n+1 == W:  D_ij = RN(kap_1,i*u_1,j), D_ij = fma(kap_m,i, u_m,j, D_ij)
 *                 for m = 2..W;  M_ij = fma(g_i, B_ij, D_ij);  the K entries of
 *                 largest |M_ij| among non-pivot rows (ties: lower index
 *                 p = j*d_k + i, column-major) become compensation values,
 *                 stored by ascending p; the rest is requantized as above with
 *                 those positions left out of both maxima (code 0); g = 1, n = 0
 *                 (delta storage is not cleared; pack clears it).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------ config */

typedef struct {
    int32_t H, dk, dv;
    int32_t unit_keyrow;    /* 0: one width per head, 1: one width per key row */
    int32_t gate_vec;       /* 0: scalar gate per head, 1: one gate per key row */
    int32_t rscale_f16;     /* 1: fp16 row scales, 0: fp32 row scales */
    int32_t cscale_f16;     /* 1: fp16 column scales, 0: none */
    int32_t window;         /* 1: requantize every step; W > 1: windowed */
    int32_t comps;          /* K fp32 compensation entries (windowed only) */
    int32_t scale_fit;      /* 0: scales refitted in the step; 1: lagged (fitted apart) */
    const uint8_t *bits;    /* H (per head) or H*dk (per key row) widths, 16 = pivot,
                               32 = fp32 (every-step mode only) */
    const float *impact;    /* NULL, or H*dk row-impact scores >= 0 (every-step mode) */
} ora_cfg;

/* Byte offsets of one head region inside a slot. */
typedef struct {
    size_t base;            /* offset of the region in the slot */
    size_t codes;           /* row bit streams, rows back to back */
    size_t rs, cs;          /* row scales, column scales (0 if absent) */
    size_t wn, g, cidx, cval, du, dkap;  /* windowed: count, gate, comps, deltas */
    size_t nrs, ncs, sr, sc; /* lagged: next row / column scales, row / column statistics */
    size_t bytes;           /* region size */
    int32_t nquant;         /* number of quantized (4/6/8-bit) rows */
} ora_head;

static int row_bits(const ora_cfg *c, int h, int i) {
    return c->unit_keyrow ? c->bits[(size_t)h * c->dk + i] : c->bits[h];
}

static size_t up(size_t x, size_t a) { return (x + a - 1) / a * a; }

/*
 * Slot layout: head regions back to back, each a multiple of 256 bytes; inside
 * a region, sections start on 16-byte boundaries in this order: codes (row i
 * takes d_v*b_i/8 bytes), row scales (if any row is quantized; d_k entries of
 * 2 or 4 bytes, 0 for pivot rows), column scales (if any row is quantized and
 * column scales are on; d_v x fp16), for lagged scales (if any row is
 * quantized): next row scales (as the row scales), next column scales (if
 * column scales are on), row statistics [d_k] fp32, column statistics [d_v]
 * fp32 (if column scales are on), then for W > 1: int32 delta count,
 * g [d_k] fp32, comp index [K] uint16, comp value [K] fp32, delta values
 * [W][d_v] fp32, delta keys [W][d_k] fp32.
 */
static size_t head_layout(const ora_cfg *c, int h, size_t base, ora_head *o) {
    memset(o, 0, sizeof *o);
    o->base = base;
    size_t p = 0;
    o->codes = p;
    int nq = 0;
    for (int i = 0; i < c->dk; ++i) {
        int b = row_bits(c, h, i);
        p += (size_t)c->dv * b / 8;
        if (b < 16) ++nq;
    }
    o->nquant = nq;
    p = up(p, 16);
    if (nq > 0) {
        o->rs = p;
        p = up(p + (size_t)c->dk * (c->rscale_f16 ? 2 : 4), 16);
        if (c->cscale_f16) {
            o->cs = p;
            p = up(p + (size_t)c->dv * 2, 16);
        }
        if (c->scale_fit == 1) {
            o->nrs = p;
            p = up(p + (size_t)c->dk * (c->rscale_f16 ? 2 : 4), 16);
            if (c->cscale_f16) {
                o->ncs = p;
                p = up(p + (size_t)c->dv * 2, 16);
            }
            o->sr = p;
            p = up(p + (size_t)c->dk * 4, 16);
            if (c->cscale_f16) {
                o->sc = p;
                p = up(p + (size_t)c->dv * 4, 16);
            }
        }
    }
    if (c->window > 1) {
        o->wn = p;      p = up(p + 4, 16);
        o->g = p;       p = up(p + (size_t)c->dk * 4, 16);
        o->cidx = p;    p = up(p + (size_t)c->comps * 2, 16);
        o->cval = p;    p = up(p + (size_t)c->comps * 4, 16);
        o->du = p;      p = up(p + (size_t)c->window * c->dv * 4, 16);
        o->dkap = p;    p = up(p + (size_t)c->window * c->dk * 4, 16);
    }
    o->bytes = up(p, 256);
    return o->bytes;
}

size_t ora_slot_bytes(const ora_cfg *c) {
    size_t base = 0;
    ora_head hd;
    for (int h = 0; h < c->H; ++h) base += head_layout(c, h, base, &hd);
    return base;
}

/* out[0..15] = base, codes, rs, cs, wn, g, cidx, cval, du, dkap, bytes, nquant,
 * nrs, ncs, sr, sc */
static void get_head(const ora_cfg *c, int h, ora_head *o);

void ora_head_layout(const ora_cfg *c, int h, uint64_t *out) {
    ora_head hd;
    get_head(c, h, &hd);
    size_t v[16] = {hd.base, hd.codes, hd.rs, hd.cs, hd.wn, hd.g, hd.cidx, hd.cval,
                    hd.du, hd.dkap, hd.bytes, (size_t)hd.nquant, hd.nrs, hd.ncs, hd.sr, hd.sc};
    for (int t = 0; t < 16; ++t) out[t] = v[t];
}

static void get_head(const ora_cfg *c, int h, ora_head *o) {
    size_t base = 0;
    for (int x = 0; x < h; ++x) base += head_layout(c, x, base, o);
    head_layout(c, h, base, o);
}

/* ------------------------------------------------------- fp16 by definition */

/* Nearest fp16 (ties to even) of a finite float, overflow to inf. */
static uint16_t f16_bits(float xf) {
    uint16_t s = signbit(xf) ? 0x8000u : 0u;
    if (isnan(xf)) return 0x7e00u;
    if (isinf(xf)) return s | 0x7c00u;
    double x = fabs((double)xf);
    if (x == 0.0) return s;
    int e;
    frexp(x, &e);              /* x = f * 2^e, f in [0.5, 1): binade exponent e-1 */
    int E = e - 1;
    if (E < -14) E = -14;      /* subnormal spacing 2^-24 */
    double m = rint(ldexp(x, 10 - E));   /* exact scaling, ties to even */
    if (m >= 2048.0) { m *= 0.5; E += 1; }
    if (E > 15) return s | 0x7c00u;
    if (m < 1024.0) return (uint16_t)(s | (uint16_t)m);
    return (uint16_t)(s | ((E + 15) << 10) | ((int)m - 1024));
}

static float f16_val(uint16_t hbits) {
    int s = hbits >> 15, E = (hbits >> 10) & 31, m = hbits & 1023;
    double v;
    if (E == 0) v = ldexp((double)m, -24);
    else if (E == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(m + 1024), E - 25);
    return (float)(s ? -v : v);
}

/* H(x): fp16 nearest-even after saturating to the largest finite fp16. */
static uint16_t H(float x) {
    if (x > 65504.0f) x = 65504.0f;
    if (x < -65504.0f) x = -65504.0f;
    return f16_bits(x);
}

/* Hup(x), x >= 0: the smallest fp16 not below x, saturating at 65504. */
static uint16_t Hup(float x) {
    uint16_t h = H(x);
    if (f16_val(h) < x && h != 0x7bffu) ++h;   /* next fp16 up (positive patterns are ordered) */
    return h;
}

void ora_f32_to_f16(const float *x, uint16_t *y, size_t n) {
    for (size_t i = 0; i < n; ++i) y[i] = f16_bits(x[i]);
}

void ora_f16_to_f32(const uint16_t *x, float *y, size_t n) {
    for (size_t i = 0; i < n; ++i) y[i] = f16_val(x[i]);
}

/* ------------------------------------------------------------- bit streams */

static uint32_t get_bits(const uint8_t *p, size_t pos, int nb) {
    uint32_t v = 0;
    for (int t = 0; t < nb; ++t) {
        size_t q = pos + (size_t)t;
        v |= (uint32_t)((p[q >> 3] >> (q & 7)) & 1u) << t;
    }
    return v;
}

static void put_bits(uint8_t *p, size_t pos, int nb, uint32_t v) {
    for (int t = 0; t < nb; ++t) {
        size_t q = pos + (size_t)t;
        uint8_t bit = (uint8_t)(1u << (q & 7));
        if ((v >> t) & 1u) p[q >> 3] |= bit;
        else p[q >> 3] &= (uint8_t)~bit;
    }
}

static float rdf(const uint8_t *p) { float f; memcpy(&f, p, 4); return f; }
static void wrf(uint8_t *p, float f) { memcpy(p, &f, 4); }
static uint16_t rdh(const uint8_t *p) { uint16_t h; memcpy(&h, p, 2); return h; }
static void wrh(uint8_t *p, uint16_t h) { memcpy(p, &h, 2); }
static int32_t rdi(const uint8_t *p) { int32_t x; memcpy(&x, p, 4); return x; }
static void wri(uint8_t *p, int32_t x) { memcpy(p, &x, 4); }

/* ------------------------------------------------------------ arithmetic */

/* csum: blocks of 8 consecutive terms as fma chains, block sums left to right. */
static float csum(const float *x, size_t xs, const float *y, int n) {
    float tot = 0.0f;
    for (int b = 0; b < n / 8; ++b) {
        float s = x[(size_t)(8 * b) * xs] * y[8 * b];
        for (int t = 1; t < 8; ++t)
            s = fmaf(x[(size_t)(8 * b + t) * xs], y[8 * b + t], s);
        tot = (b == 0) ? s : tot + s;
    }
    return tot;
}

static int qmax_of(int b) { return (1 << (b - 1)) - 1; }

/* Unpacked view of one head: codes n_ij (pivot rows: fp16 pattern), scales. */
typedef struct {
    int32_t *n;      /* dk*dv */
    uint16_t *hv;    /* dk*dv, pivot rows */
    float *fv;       /* dk*dv, fp32 rows */
    int *bw;         /* dk widths */
    float *r, *c;    /* dk, dv */
    float *g;        /* dk (windowed) */
    int32_t nd;      /* delta count (windowed) */
    uint16_t *cidx;  /* K */
    float *cval;     /* K */
    float *du, *dkap;/* W*dv, W*dk */
    float *nr, *nc;  /* lagged: next row / column scales (dk, dv) */
    float *sR, *sC;  /* lagged: row / column statistics (dk, dv) */
} ora_unit;

static void unit_alloc(const ora_cfg *c, ora_unit *u) {
    size_t e = (size_t)c->dk * c->dv;
    u->n = calloc(e, sizeof(int32_t));
    u->hv = calloc(e, sizeof(uint16_t));
    u->fv = calloc(e, sizeof(float));
    u->bw = calloc((size_t)c->dk, sizeof(int));
    u->r = calloc((size_t)c->dk, sizeof(float));
    u->c = calloc((size_t)c->dv, sizeof(float));
    u->g = calloc((size_t)c->dk, sizeof(float));
    u->cidx = calloc((size_t)(c->comps + 1), sizeof(uint16_t));
    u->cval = calloc((size_t)(c->comps + 1), sizeof(float));
    u->du = calloc((size_t)c->window * c->dv, sizeof(float));
    u->dkap = calloc((size_t)c->window * c->dk, sizeof(float));
    u->nr = calloc((size_t)c->dk, sizeof(float));
    u->nc = calloc((size_t)c->dv, sizeof(float));
    u->sR = calloc((size_t)c->dk, sizeof(float));
    u->sC = calloc((size_t)c->dv, sizeof(float));
    u->nd = 0;
}

static void unit_free(ora_unit *u) {
    free(u->n); free(u->hv); free(u->fv); free(u->bw); free(u->r); free(u->c); free(u->g);
    free(u->cidx); free(u->cval); free(u->du); free(u->dkap);
    free(u->nr); free(u->nc); free(u->sR); free(u->sC);
}

static void unit_read(const ora_cfg *c, int h, const uint8_t *slot, ora_unit *u) {
    ora_head hd;
    get_head(c, h, &hd);
    const uint8_t *R = slot + hd.base;
    size_t rowoff = hd.codes;
    for (int i = 0; i < c->dk; ++i) {
        int b = row_bits(c, h, i);
        u->bw[i] = b;
        for (int j = 0; j < c->dv; ++j) {
            uint32_t raw = get_bits(R + rowoff, (size_t)j * b, b);
            size_t e = (size_t)i * c->dv + j;
            if (b == 32) { memcpy(&u->fv[e], &raw, 4); u->n[e] = 0; }
            else if (b == 16) { u->hv[e] = (uint16_t)raw; u->n[e] = 0; }
            else u->n[e] = (int32_t)raw - (1 << (b - 1));
        }
        rowoff += (size_t)c->dv * b / 8;
    }
    for (int i = 0; i < c->dk; ++i) {
        if (hd.nquant == 0) u->r[i] = 0.0f;
        else if (c->rscale_f16) u->r[i] = f16_val(rdh(R + hd.rs + 2 * (size_t)i));
        else u->r[i] = rdf(R + hd.rs + 4 * (size_t)i);
    }
    for (int j = 0; j < c->dv; ++j)
        u->c[j] = (hd.nquant > 0 && c->cscale_f16) ? f16_val(rdh(R + hd.cs + 2 * (size_t)j)) : 1.0f;
    if (c->scale_fit == 1 && hd.nquant > 0) {
        for (int i = 0; i < c->dk; ++i) {
            u->nr[i] = c->rscale_f16 ? f16_val(rdh(R + hd.nrs + 2 * (size_t)i)) : rdf(R + hd.nrs + 4 * (size_t)i);
            u->sR[i] = rdf(R + hd.sr + 4 * (size_t)i);
        }
        for (int j = 0; j < c->dv; ++j) {
            u->nc[j] = c->cscale_f16 ? f16_val(rdh(R + hd.ncs + 2 * (size_t)j)) : 1.0f;
            u->sC[j] = c->cscale_f16 ? rdf(R + hd.sc + 4 * (size_t)j) : 0.0f;
        }
    }
    if (c->window > 1) {
        u->nd = rdi(R + hd.wn);
        for (int i = 0; i < c->dk; ++i) u->g[i] = rdf(R + hd.g + 4 * (size_t)i);
        for (int t = 0; t < c->comps; ++t) {
            u->cidx[t] = rdh(R + hd.cidx + 2 * (size_t)t);
            u->cval[t] = rdf(R + hd.cval + 4 * (size_t)t);
        }
        for (size_t t = 0; t < (size_t)c->window * c->dv; ++t) u->du[t] = rdf(R + hd.du + 4 * t);
        for (size_t t = 0; t < (size_t)c->window * c->dk; ++t) u->dkap[t] = rdf(R + hd.dkap + 4 * t);
    }
}

static void unit_write(const ora_cfg *c, int h, uint8_t *slot, const ora_unit *u) {
    ora_head hd;
    get_head(c, h, &hd);
    uint8_t *R = slot + hd.base;
    size_t rowoff = hd.codes;
    for (int i = 0; i < c->dk; ++i) {
        int b = row_bits(c, h, i);
        for (int j = 0; j < c->dv; ++j) {
            size_t e = (size_t)i * c->dv + j;
            uint32_t raw;
            if (b == 32) memcpy(&raw, &u->fv[e], 4);
            else if (b == 16) raw = u->hv[e];
            else raw = (uint32_t)(u->n[e] + (1 << (b - 1)));
            put_bits(R + rowoff, (size_t)j * b, b, raw);
        }
        rowoff += (size_t)c->dv * b / 8;
    }
    if (hd.nquant > 0) {
        for (int i = 0; i < c->dk; ++i) {
            if (c->rscale_f16) wrh(R + hd.rs + 2 * (size_t)i, H(u->r[i]));
            else wrf(R + hd.rs + 4 * (size_t)i, u->r[i]);
        }
        if (c->cscale_f16)
            for (int j = 0; j < c->dv; ++j) wrh(R + hd.cs + 2 * (size_t)j, H(u->c[j]));
        if (c->scale_fit == 1) {
            for (int i = 0; i < c->dk; ++i) {
                if (c->rscale_f16) wrh(R + hd.nrs + 2 * (size_t)i, H(u->nr[i]));
                else wrf(R + hd.nrs + 4 * (size_t)i, u->nr[i]);
                wrf(R + hd.sr + 4 * (size_t)i, u->sR[i]);
            }
            if (c->cscale_f16)
                for (int j = 0; j < c->dv; ++j) {
                    wrh(R + hd.ncs + 2 * (size_t)j, H(u->nc[j]));
                    wrf(R + hd.sc + 4 * (size_t)j, u->sC[j]);
                }
        }
    }
    if (c->window > 1) {
        wri(R + hd.wn, u->nd);
        for (int i = 0; i < c->dk; ++i) wrf(R + hd.g + 4 * (size_t)i, u->g[i]);
        for (int t = 0; t < c->comps; ++t) {
            wrh(R + hd.cidx + 2 * (size_t)t, u->cidx[t]);
            wrf(R + hd.cval + 4 * (size_t)t, u->cval[t]);
        }
        for (size_t t = 0; t < (size_t)c->window * c->dv; ++t) wrf(R + hd.du + 4 * t, u->du[t]);
        for (size_t t = 0; t < (size_t)c->window * c->dk; ++t) wrf(R + hd.dkap + 4 * t, u->dkap[t]);
    }
}

/* Base dequantization B_ij = RN(n_ij * r_i * c_j) (n*r is exact) and pivots;
 * with_comps: compensation entries overwrite their positions. */
static void dequant_base(const ora_cfg *c, const ora_unit *u, float *B, int with_comps) {
    for (int i = 0; i < c->dk; ++i)
        for (int j = 0; j < c->dv; ++j) {
            size_t e = (size_t)i * c->dv + j;
            if (u->bw[i] == 32) B[e] = u->fv[e];
            else if (u->bw[i] == 16) B[e] = f16_val(u->hv[e]);
            else B[e] = ((float)u->n[e] * u->r[i]) * u->c[j];
        }
    if (c->window > 1 && with_comps)
        for (int t = 0; t < c->comps; ++t) {
            int i = u->cidx[t] % c->dk, j = u->cidx[t] / c->dk;
            B[(size_t)i * c->dv + j] = u->cval[t];
        }
}

/* Requantize into u (codes, pivots, scales) the state whose column j is
 * M[., j] * s[j] (s == NULL: all ones, M is the state itself).  skip[e] != 0
 * excludes an entry. */
/* Row-impact weights of head h (NULL without impact scores). */
static float *impact_weights(const ora_cfg *c, int h) {
    if (!c->impact) return NULL;
    float *w = malloc(sizeof(float) * (size_t)c->dk);
    double mx = 0.0;
    for (int i = 0; i < c->dk; ++i) {
        double v = c->impact[(size_t)h * c->dk + i];
        if (v > mx) mx = v;
    }
    for (int i = 0; i < c->dk; ++i)
        w[i] = mx > 0.0 ? (float)sqrt((double)c->impact[(size_t)h * c->dk + i] / mx) : 1.0f;
    return w;
}

static void requantize(const ora_cfg *c, int h, ora_unit *u, const float *M, const float *s,
                       const uint8_t *skip) {
    int dk = c->dk, dv = c->dv;
    float *f = malloc(sizeof(float) * (size_t)dv);
    float *Z = malloc(sizeof(float) * (size_t)dk * dv);
    float *wi = impact_weights(c, h);
    for (int j = 0; j < dv; ++j) {
        if (!c->cscale_f16) { u->c[j] = 1.0f; f[j] = 1.0f; continue; }
        float sj = s ? s[j] : 1.0f;
        float C = 0.0f;
        for (int i = 0; i < dk; ++i) {
            size_t e = (size_t)i * dv + j;
            if (u->bw[i] >= 16 || (skip && skip[e])) continue;
            float a = wi ? wi[i] * fabsf(M[e]) : fabsf(M[e]);
            if (a > C) C = a;
        }
        u->sC[j] = C * sj;
        u->c[j] = f16_val(H(C * sj));
        f[j] = u->c[j] > 0.0f ? sj / u->c[j] : 0.0f;
    }
    for (int i = 0; i < dk; ++i) {
        if (u->bw[i] >= 16) {
            /* pivot rows keep the fp16 of the state, fp32 rows the state itself */
            u->r[i] = 0.0f;
            for (int j = 0; j < dv; ++j) {
                size_t e = (size_t)i * dv + j;
                float sj = s ? s[j] : 1.0f;
                if (u->bw[i] == 32) u->fv[e] = M[e] * sj;
                else u->hv[e] = H(M[e] * sj);
                u->n[e] = 0;
            }
            continue;
        }
        float R = 0.0f;
        for (int j = 0; j < dv; ++j) {
            size_t e = (size_t)i * dv + j;
            Z[e] = (skip && skip[e]) ? 0.0f : (c->cscale_f16 ? M[e] * f[j] : M[e]);
            float a = fabsf(Z[e]);
            if (a > R) R = a;
        }
        int qm = qmax_of(u->bw[i]);
        u->sR[i] = R;
        float rq = R / (float)qm;
        u->r[i] = c->rscale_f16 ? f16_val(Hup(rq)) : rq;
        float ir = u->r[i] > 0.0f ? 1.0f / u->r[i] : 0.0f;
        if (isinf(ir)) ir = 0.0f;
        for (int j = 0; j < dv; ++j) {
            size_t e = (size_t)i * dv + j;
            /* the product of two floats is exact in double; rint rounds ties to even */
            double x = rint((double)Z[e] * (double)ir);
            if (x > qm) x = qm;
            if (x < -qm) x = -qm;
            u->n[e] = (skip && skip[e]) ? 0 : (int32_t)x;
            u->hv[e] = 0;
        }
    }
    free(f);
    free(Z);
    free(wi);
}

/* Lagged scales: quantize the working state M'' (column j in units of s[j])
 * with the next scales u->nr, u->nc fitted to the previous state, clamping to
 * +-qmax; record the refit statistics of this state (the every-step refit's
 * column absmax and row absmax); the next scales become the scales of the
 * codes. */
static void quantize_lagged(const ora_cfg *c, ora_unit *u, const float *M, const float *s) {
    int dk = c->dk, dv = c->dv;
    float *f = malloc(sizeof(float) * (size_t)dv);
    float *ff = malloc(sizeof(float) * (size_t)dv);
    for (int j = 0; j < dv; ++j) {
        if (!c->cscale_f16) { f[j] = 1.0f; ff[j] = 1.0f; u->sC[j] = 0.0f; continue; }
        float C = 0.0f;
        for (int i = 0; i < dk; ++i) {
            if (u->bw[i] >= 16) continue;
            float a = fabsf(M[(size_t)i * dv + j]);
            if (a > C) C = a;
        }
        u->sC[j] = C * s[j];
        float cfit = f16_val(H(u->sC[j]));
        ff[j] = cfit > 0.0f ? s[j] / cfit : 0.0f;
        f[j] = u->nc[j] > 0.0f ? s[j] / u->nc[j] : 0.0f;
    }
    for (int i = 0; i < dk; ++i) {
        if (u->bw[i] >= 16) {
            u->r[i] = 0.0f;
            u->sR[i] = 0.0f;
            for (int j = 0; j < dv; ++j) {
                size_t e = (size_t)i * dv + j;
                if (u->bw[i] == 32) u->fv[e] = M[e] * s[j];
                else u->hv[e] = H(M[e] * s[j]);
                u->n[e] = 0;
            }
            continue;
        }
        int qm = qmax_of(u->bw[i]);
        float ir = u->nr[i] > 0.0f ? 1.0f / u->nr[i] : 0.0f;
        if (isinf(ir)) ir = 0.0f;
        float R = 0.0f;
        for (int j = 0; j < dv; ++j) {
            size_t e = (size_t)i * dv + j;
            float Zf = c->cscale_f16 ? M[e] * ff[j] : M[e];
            if (fabsf(Zf) > R) R = fabsf(Zf);
            float Z = c->cscale_f16 ? M[e] * f[j] : M[e];
            double x = rint((double)Z * (double)ir);
            if (x > qm) x = qm;
            if (x < -qm) x = -qm;
            u->n[e] = (int32_t)x;
            u->hv[e] = 0;
        }
        u->sR[i] = R;
        u->r[i] = u->nr[i];
    }
    for (int j = 0; j < dv; ++j) u->c[j] = c->cscale_f16 ? u->nc[j] : 1.0f;
    free(f);
    free(ff);
}

/* Top-K |M| among entries of non-pivot rows; ties to the lower column-major
 * index p = j*dk + i.  Stored by ascending p. */
typedef struct { float mag; uint32_t idx; } ora_ent;
static int ent_cmp(const void *pa, const void *pb) {
    const ora_ent *a = pa, *b = pb;
    if (a->mag != b->mag) return a->mag > b->mag ? -1 : 1;
    return a->idx < b->idx ? -1 : (a->idx > b->idx);
}
static int idx_cmp(const void *pa, const void *pb) {
    uint16_t a = *(const uint16_t *)pa, b = *(const uint16_t *)pb;
    return (a > b) - (a < b);
}

static void select_comps(const ora_cfg *c, ora_unit *u, const float *M, uint8_t *skip) {
    size_t e = (size_t)c->dk * c->dv, m = 0;
    ora_ent *all = malloc(sizeof(ora_ent) * e);
    for (int i = 0; i < c->dk; ++i) {
        if (u->bw[i] >= 16) continue;
        for (int j = 0; j < c->dv; ++j) {
            all[m].mag = fabsf(M[(size_t)i * c->dv + j]);
            all[m].idx = (uint32_t)((size_t)j * c->dk + i);
            ++m;
        }
    }
    qsort(all, m, sizeof(ora_ent), ent_cmp);
    memset(skip, 0, e);
    for (int t = 0; t < c->comps; ++t) u->cidx[t] = (uint16_t)all[t].idx;
    qsort(u->cidx, (size_t)c->comps, sizeof(uint16_t), idx_cmp);
    for (int t = 0; t < c->comps; ++t) {
        size_t x = (size_t)(u->cidx[t] % c->dk) * c->dv + u->cidx[t] / c->dk;
        u->cval[t] = M[x];
        skip[x] = 1;
    }
    free(all);
}

/* ------------------------------------------------------------- public API */

/* Empty slot: all bytes zero, cumulative gates 1 (windowed). */
void ora_slot_init(const ora_cfg *c, uint8_t *slot) {
    memset(slot, 0, ora_slot_bytes(c));
    if (c->window > 1)
        for (int h = 0; h < c->H; ++h) {
            ora_head hd;
            get_head(c, h, &hd);
            for (int i = 0; i < c->dk; ++i) wrf(slot + hd.base + hd.g + 4 * (size_t)i, 1.0f);
        }
}

/* Current state of head h as fp32 [dk*dv]: dequantized base, or for W > 1 the
 * materialized M = fma(g, B, D) of the base and the stored deltas. */
void ora_unpack_head(const ora_cfg *c, int h, const uint8_t *slot, float *M) {
    ora_unit u;
    unit_alloc(c, &u);
    unit_read(c, h, slot, &u);
    dequant_base(c, &u, M, 1);
    if (c->window > 1 && u.nd > 0) {
        for (int i = 0; i < c->dk; ++i)
            for (int j = 0; j < c->dv; ++j) {
                size_t e = (size_t)i * c->dv + j;
                float D = u.dkap[i] * u.du[j];
                for (int m = 1; m < u.nd; ++m)
                    D = fmaf(u.dkap[(size_t)m * c->dk + i], u.du[(size_t)m * c->dv + j], D);
                M[e] = fmaf(u.g[i], M[e], D);
            }
    }
    unit_free(&u);
}

/* Quantize fp32 state M [dk*dv] into head h (windowed: comps, g = 1, n = 0). */
void ora_pack_head(const ora_cfg *c, int h, uint8_t *slot, const float *M) {
    ora_unit u;
    unit_alloc(c, &u);
    unit_read(c, h, slot, &u);
    uint8_t *skip = NULL;
    if (c->window > 1) {
        skip = calloc((size_t)c->dk * c->dv, 1);
        select_comps(c, &u, M, skip);
        for (int i = 0; i < c->dk; ++i) u.g[i] = 1.0f;
        u.nd = 0;
        memset(u.du, 0, sizeof(float) * (size_t)c->window * c->dv);
        memset(u.dkap, 0, sizeof(float) * (size_t)c->window * c->dk);
    }
    requantize(c, h, &u, M, NULL, skip);
    if (c->scale_fit == 1) {
        /* lagged scales: no next scales yet, so the next step refits in the step */
        memset(u.nr, 0, sizeof(float) * (size_t)c->dk);
        memset(u.nc, 0, sizeof(float) * (size_t)c->dv);
    }
    unit_write(c, h, slot, &u);
    free(skip);
    unit_free(&u);
}

/* One decode step of head h.  q, k: [dk]; v: [dv]; a: [dk] if gate_vec else
 * [1]; beta scalar.  Writes o [dv] and updates the head region in place. */
void ora_step_head(const ora_cfg *c, int h, uint8_t *slot, const float *q, const float *k,
                   const float *v, const float *a, float beta, float *o) {
    int dk = c->dk, dv = c->dv;
    size_t e = (size_t)dk * dv;
    ora_unit u;
    unit_alloc(c, &u);
    unit_read(c, h, slot, &u);
    float *ai = malloc(sizeof(float) * (size_t)dk);
    for (int i = 0; i < dk; ++i) ai[i] = c->gate_vec ? a[i] : a[0];
    float *M = malloc(sizeof(float) * e);

    if (c->window == 1) {
        float *A = malloc(sizeof(float) * e);
        float *sc = malloc(sizeof(float) * (size_t)dv);
        float *is = malloc(sizeof(float) * (size_t)dv);
        /* u.c is 1 where the head has no column scales */
        for (int j = 0; j < dv; ++j) {
            sc[j] = u.c[j] > 0.0f ? u.c[j] : 1.0f;
            is[j] = 1.0f / sc[j];
        }
        for (int i = 0; i < dk; ++i) {
            float gi = ai[i] * u.r[i];
            for (int j = 0; j < dv; ++j) {
                size_t x = (size_t)i * dv + j;
                if (u.bw[i] == 32) A[x] = ai[i] * u.fv[x];
                else if (u.bw[i] == 16) A[x] = (ai[i] * f16_val(u.hv[x])) * is[j];
                else A[x] = (float)u.n[x] * gi;
            }
        }
        for (int j = 0; j < dv; ++j) {
            float w = sc[j] * csum(A + j, (size_t)dv, k, dk);
            float uj = beta * (v[j] - w);
            float us = uj * is[j];
            for (int i = 0; i < dk; ++i) {
                size_t x = (size_t)i * dv + j;
                M[x] = fmaf(k[i], us, A[x]);
            }
        }
        for (int j = 0; j < dv; ++j) o[j] = sc[j] * csum(M + j, (size_t)dv, q, dk);
        int fitted = 0;   /* lagged scales: some quantized row has a next scale */
        if (c->scale_fit == 1)
            for (int i = 0; i < dk; ++i) fitted |= u.bw[i] < 16 && u.nr[i] > 0.0f;
        if (fitted) quantize_lagged(c, &u, M, sc);
        else requantize(c, h, &u, M, sc, NULL);
        free(A);
        free(sc);
        free(is);
    } else {
        int W = c->window, n = u.nd;
        float *B = malloc(sizeof(float) * e);
        float *kg = malloc(sizeof(float) * (size_t)dk);
        float *qg = malloc(sizeof(float) * (size_t)dk);
        float *ck = malloc(sizeof(float) * (size_t)(W + 1));
        float *cq = malloc(sizeof(float) * (size_t)(W + 1));
        float *un = malloc(sizeof(float) * (size_t)dv);
        float *Bc = malloc(sizeof(float) * e);
        dequant_base(c, &u, B, 0);
        dequant_base(c, &u, Bc, 1);
        for (int m = 0; m < n; ++m)
            for (int i = 0; i < dk; ++i) u.dkap[(size_t)m * dk + i] *= ai[i];
        for (int i = 0; i < dk; ++i) {
            u.g[i] = u.g[i] * ai[i];
            kg[i] = u.g[i] * k[i];
            qg[i] = u.g[i] * q[i];
        }
        for (int m = 0; m < n; ++m) ck[m] = csum(u.dkap + (size_t)m * dk, 1, k, dk);
        for (int j = 0; j < dv; ++j) {
            float w = csum(B + j, (size_t)dv, kg, dk);
            for (int t = 0; t < c->comps; ++t)
                if (u.cidx[t] / dk == j) w = fmaf(u.cval[t], kg[u.cidx[t] % dk], w);
            for (int m = 0; m < n; ++m) w = fmaf(u.du[(size_t)m * dv + j], ck[m], w);
            un[j] = beta * (v[j] - w);
        }
        for (int j = 0; j < dv; ++j) u.du[(size_t)n * dv + j] = un[j];
        for (int i = 0; i < dk; ++i) u.dkap[(size_t)n * dk + i] = k[i];
        ++n;
        for (int m = 0; m < n; ++m) cq[m] = csum(u.dkap + (size_t)m * dk, 1, q, dk);
        for (int j = 0; j < dv; ++j) {
            float p = csum(B + j, (size_t)dv, qg, dk);
            for (int t = 0; t < c->comps; ++t)
                if (u.cidx[t] / dk == j) p = fmaf(u.cval[t], qg[u.cidx[t] % dk], p);
            for (int m = 0; m < n; ++m) p = fmaf(u.du[(size_t)m * dv + j], cq[m], p);
            o[j] = p;
        }
        u.nd = n;
        if (n == W) {
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) {
                    size_t x = (size_t)i * dv + j;
                    float D = u.dkap[i] * u.du[j];
                    for (int m = 1; m < W; ++m)
                        D = fmaf(u.dkap[(size_t)m * dk + i], u.du[(size_t)m * dv + j], D);
                    M[x] = fmaf(u.g[i], Bc[x], D);
                }
            uint8_t *skip = calloc(e, 1);
            select_comps(c, &u, M, skip);
            requantize(c, h, &u, M, NULL, skip);
            for (int i = 0; i < dk; ++i) u.g[i] = 1.0f;
            u.nd = 0;   /* the stored deltas are left as they are: only n counts */
            free(skip);
        }
        free(B); free(Bc); free(kg); free(qg); free(ck); free(cq); free(un);
    }
    unit_write(c, h, slot, &u);
    free(M);
    free(ai);
    unit_free(&u);
}

/* Lagged scales: the next scales of head h from its statistics. */
void ora_fit_head(const ora_cfg *c, int h, uint8_t *slot) {
    if (c->scale_fit != 1) return;
    ora_unit u;
    unit_alloc(c, &u);
    unit_read(c, h, slot, &u);
    for (int i = 0; i < c->dk; ++i) {
        if (u.bw[i] >= 16) { u.nr[i] = 0.0f; continue; }
        float rq = u.sR[i] / (float)qmax_of(u.bw[i]);
        u.nr[i] = c->rscale_f16 ? f16_val(Hup(rq)) : rq;
    }
    for (int j = 0; j < c->dv; ++j) u.nc[j] = c->cscale_f16 ? f16_val(H(u.sC[j])) : 1.0f;
    unit_write(c, h, slot, &u);
    unit_free(&u);
}

/* Unquantized fp32 step on M [dk*dv] in place: A = RN(a_i*M_ij), then the same
 * read / delta / write / output as the quantized step. */
void ora_step_f32(int dk, int dv, int gate_vec, float *M, const float *q, const float *k,
                  const float *v, const float *a, float beta, float *o) {
    size_t e = (size_t)dk * dv;
    float *A = malloc(sizeof(float) * e);
    for (int i = 0; i < dk; ++i) {
        float ai = gate_vec ? a[i] : a[0];
        for (int j = 0; j < dv; ++j) A[(size_t)i * dv + j] = ai * M[(size_t)i * dv + j];
    }
    for (int j = 0; j < dv; ++j) {
        float w = csum(A + j, (size_t)dv, k, dk);
        float uj = beta * (v[j] - w);
        for (int i = 0; i < dk; ++i) {
            size_t x = (size_t)i * dv + j;
            M[x] = fmaf(k[i], uj, A[x]);
        }
    }
    for (int j = 0; j < dv; ++j) o[j] = csum(M + j, (size_t)dv, q, dk);
    free(A);
}

/* The same recurrence in fp64, plain sums (for closed forms and Proposition 1). */
void ora_step_f64(int dk, int dv, int gate_vec, double *M, const double *q, const double *k,
                  const double *v, const double *a, double beta, double *o) {
    for (int i = 0; i < dk; ++i) {
        double ai = gate_vec ? a[i] : a[0];
        for (int j = 0; j < dv; ++j) M[(size_t)i * dv + j] *= ai;
    }
    for (int j = 0; j < dv; ++j) {
        double w = 0.0;
        for (int i = 0; i < dk; ++i) w += M[(size_t)i * dv + j] * k[i];
        double uj = beta * (v[j] - w);
        for (int i = 0; i < dk; ++i) M[(size_t)i * dv + j] += k[i] * uj;
    }
    for (int j = 0; j < dv; ++j) {
        double s = 0.0;
        for (int i = 0; i < dk; ++i) s += M[(size_t)i * dv + j] * q[i];
        o[j] = s;
    }
}

/* Exposed pieces for the pins: the canonical sum. */
float ora_csum(const float *x, const float *y, int n) { return csum(x, 1, y, n); }
