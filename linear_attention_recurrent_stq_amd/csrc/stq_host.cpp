// Host side of the C ABI (include/stq.h): configuration checks, slot layout,
// pool carving and kernel launches.  Nothing here synchronizes the device.
//
// Slot layout (one request, one layer): the H head regions back to back, each
// a multiple of 256 bytes.  Inside a region, sections start on 16-byte
// boundaries: code rows (row i takes d_v*b_i/8 bytes; fp16 patterns for
// pivot rows), row scales [d_k] (fp16 or fp32) and column scales [d_v] fp16
// when the head has a quantized row, then for the windowed mode the delta
// count, cumulative gate g [d_k], compensation indices [K] uint16 and values
// [K] fp32, delta values [W][d_v] and delta keys [W][d_k] (fp32); for lagged
// scales (when the head has a quantized row) the next row scales, next column
// scales, row statistics [d_k] fp32 and column statistics [d_v] fp32.
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "stq.h"

#include "stq_internal.h"

struct stq_layout {
    stq_config cfg;                     // unit_bits cleared; widths live in `bits`
    bool mixed = false;                 // some head has rows of different widths
    int step_mix = 0;                   // 0 none; 1 only 4-bit + pivot row heads; 2 other
    std::vector<uint8_t> bits;          // H or H*d_k unit widths
    std::vector<stq::HeadDesc> heads;   // [H]
    std::vector<uint32_t> rows;         // [H*d_k] row table
    std::vector<uint32_t> groups;       // step-kernel head groups (h1 | h2 << 16)
    std::vector<float> omega;           // row-impact weights [H*d_k] (empty: none)
    std::vector<uint8_t> table;         // device image: heads, rows, groups, weights, (windowed)
                                        // window-end flag; 256-B padded
    size_t flag_off = 0;                // windowed: byte offset of the window-end flag (8 bytes)
    size_t slot_bytes = 0;
};

namespace {

thread_local std::string g_err;
// Windowed decode calls of the process, numbered from 1: the token a call's
// in-window step leaves in the pool's window-end flag.
std::atomic<uint64_t> g_token{0};

stq_status fail(stq_status s, const std::string &msg) {
    g_err = msg;
    return s;
}

size_t up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

stq_status check_cfg(const stq_config *c) {
    if (!c) return fail(STQ_ERR_INVALID, "config is NULL");
    if (c->H < 1 || c->H > 4096) return fail(STQ_ERR_INVALID, "H must be in [1, 4096]");
    if ((c->d_k != 64 && c->d_k != 128) || (c->d_v != 64 && c->d_v != 128))
        return fail(STQ_ERR_UNSUPPORTED, "d_k and d_v must each be 64 or 128");
    if (c->unit != STQ_UNIT_HEAD && c->unit != STQ_UNIT_KEYROW)
        return fail(STQ_ERR_INVALID, "unit must be STQ_UNIT_HEAD or STQ_UNIT_KEYROW");
    if (c->gate != STQ_GATE_SCALAR && c->gate != STQ_GATE_KEYVEC)
        return fail(STQ_ERR_INVALID, "gate must be STQ_GATE_SCALAR or STQ_GATE_KEYVEC");
    if (c->row_scale != STQ_F16 && c->row_scale != STQ_F32)
        return fail(STQ_ERR_INVALID, "row_scale must be STQ_F16 or STQ_F32");
    if (c->col_scale != STQ_F16 && c->col_scale != STQ_NONE)
        return fail(STQ_ERR_INVALID, "col_scale must be STQ_F16 or STQ_NONE");
    if (c->io_dtype != STQ_BF16 && c->io_dtype != STQ_F32)
        return fail(STQ_ERR_INVALID, "io_dtype must be STQ_BF16 or STQ_F32");
    if (c->window < 1) return fail(STQ_ERR_INVALID, "window must be >= 1");
    if (c->window > 16) return fail(STQ_ERR_UNSUPPORTED, "window must be <= 16");
    if (c->comps < 0 || c->comps > 1024) return fail(STQ_ERR_INVALID, "comps must be in [0, 1024]");
    if (c->window == 1 && c->comps != 0)
        return fail(STQ_ERR_INVALID, "compensation entries need the windowed mode (window > 1)");
    if (c->scale_fit != STQ_FIT_STEP && c->scale_fit != STQ_FIT_LAGGED)
        return fail(STQ_ERR_INVALID, "scale_fit must be STQ_FIT_STEP or STQ_FIT_LAGGED");
    if (c->scale_fit == STQ_FIT_LAGGED && c->window != 1)
        return fail(STQ_ERR_UNSUPPORTED, "lagged scales need the every-step mode (window 1)");
    if (c->row_impact) {
        if (c->window != 1 || c->scale_fit != STQ_FIT_STEP)
            return fail(STQ_ERR_UNSUPPORTED, "row-impact scores need the every-step mode with scales fitted in the step");
        const size_t nr = (size_t)c->H * (size_t)c->d_k;
        for (size_t i = 0; i < nr; ++i)
            if (!(c->row_impact[i] >= 0.0f) || !std::isfinite(c->row_impact[i])) {
                char m[96];
                std::snprintf(m, sizeof m, "row_impact[%zu] is negative or not finite", i);
                return fail(STQ_ERR_INVALID, m);
            }
    }
    if (!c->unit_bits) return fail(STQ_ERR_INVALID, "unit_bits is NULL");
    const size_t n = (size_t)c->H * (c->unit == STQ_UNIT_KEYROW ? c->d_k : 1);
    for (size_t i = 0; i < n; ++i) {
        const uint8_t b = c->unit_bits[i];
        if (b != 4 && b != 6 && b != 8 && b != 16 && b != 32) {
            char m[96];
            std::snprintf(m, sizeof m, "unit_bits[%zu] = %u is not in {4,6,8,16,32}", i, (unsigned)b);
            return fail(STQ_ERR_INVALID, m);
        }
        if (b == 32 && c->window > 1)
            return fail(STQ_ERR_UNSUPPORTED, "fp32 units (width 32) need the every-step mode (window 1)");
    }
    if (c->unit == STQ_UNIT_KEYROW) {
        // an fp32 unit is a whole head: its key rows are all fp32 or none is
        for (int h = 0; h < c->H; ++h) {
            int n32 = 0;
            for (int i = 0; i < c->d_k; ++i) n32 += c->unit_bits[(size_t)h * c->d_k + i] == 32;
            if (n32 != 0 && n32 != c->d_k)
                return fail(STQ_ERR_UNSUPPORTED, "fp32 units (width 32) must cover whole heads");
        }
    }
    return STQ_OK;
}

stq_status check_pool(const stq_pool *p) {
    if (!p || !p->layout || !p->base) return fail(STQ_ERR_INVALID, "pool is NULL or not allocated");
    if (p->slots < 0) return fail(STQ_ERR_INVALID, "pool has a negative slot count");
    return STQ_OK;
}

stq::Args base_args(const stq_pool *p, int32_t B, const int32_t *ids) {
    const stq_layout *L = p->layout;
    stq::Args a{};
    uint8_t *base = static_cast<uint8_t *>(p->base);
    a.slots = base + L->table.size();
    a.heads = reinterpret_cast<const stq::HeadDesc *>(base);
    a.rows = reinterpret_cast<const uint32_t *>(base + sizeof(stq::HeadDesc) * L->heads.size());
    a.groups = a.rows + L->rows.size();
    a.ngroups = (int32_t)L->groups.size();
    a.omega = L->omega.empty() ? nullptr : reinterpret_cast<const float *>(a.groups + L->groups.size());
    a.slot_bytes = L->slot_bytes;
    a.slot_ids = ids;
    a.B = B;
    a.H = L->cfg.H;
    a.nslots = p->slots;
    a.io_bf16 = L->cfg.io_dtype == STQ_BF16;
    a.gate_vec = L->cfg.gate == STQ_GATE_KEYVEC;
    a.rs16 = L->cfg.row_scale == STQ_F16;
    a.cs16 = L->cfg.col_scale == STQ_F16;
    a.window = L->cfg.window;
    a.comps = L->cfg.comps;
    a.lagged = L->cfg.scale_fit == STQ_FIT_LAGGED;
    if (L->cfg.window > 1) a.end_flag = reinterpret_cast<uint64_t *>(base + L->flag_off);
    return a;
}

stq_status launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(STQ_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
    return STQ_OK;
}

// Every id in [0, slots), none twice (host ids).
stq_status check_ids_host(int32_t slots, int32_t B, const int32_t *ids) {
    std::vector<uint8_t> seen((size_t)slots, 0);
    for (int32_t b = 0; b < B; ++b) {
        const int32_t s = ids[b];
        char m[128];
        if (s < 0 || s >= slots) {
            std::snprintf(m, sizeof m, "slot id %d at position %d is outside [0, %d)", s, b, slots);
            return fail(STQ_ERR_INVALID, m);
        }
        if (seen[(size_t)s]) {
            std::snprintf(m, sizeof m, "slot id %d at position %d appears twice in the batch", s, b);
            return fail(STQ_ERR_INVALID, m);
        }
        seen[(size_t)s] = 1;
    }
    return STQ_OK;
}

stq_status check_batch(const stq_pool *pool, int32_t B, const int32_t *ids) {
    if (stq_status s = check_pool(pool)) return s;
    if (B < 0) return fail(STQ_ERR_INVALID, "B must be >= 0");
    if (B > pool->slots) return fail(STQ_ERR_INVALID, "B exceeds the pool's slot count");
    if (B > 0 && !ids) return fail(STQ_ERR_INVALID, "slot ids are NULL");
    if (B > 0 && !aligned(ids, 4)) return fail(STQ_ERR_ALIGN, "slot ids must be 4-byte aligned");
#if STQ_DEBUG_VALIDATE
    // debug builds: copy the ids back (a synchronizing copy) and check them
    if (B > 0) {
        std::vector<int32_t> h((size_t)B);
        const hipError_t e = hipMemcpy(h.data(), ids, sizeof(int32_t) * (size_t)B, hipMemcpyDeviceToHost);
        if (e != hipSuccess)
            return fail(STQ_ERR_DEVICE, std::string("slot id copy: ") + hipGetErrorString(e));
        if (stq_status s = check_ids_host(pool->slots, B, h.data())) return s;
    }
#endif
    return STQ_OK;
}

}  // namespace

namespace stq {
// The last-error text of this thread, for the other host sources.
void set_error(const std::string &msg) { g_err = msg; }
}  // namespace stq

extern "C" {

const char *stq_status_string(stq_status s) {
    switch (s) {
        case STQ_OK: return "ok";
        case STQ_ERR_INVALID: return "invalid argument";
        case STQ_ERR_UNSUPPORTED: return "unsupported configuration";
        case STQ_ERR_TOO_SMALL: return "buffer too small";
        case STQ_ERR_ALIGN: return "misaligned pointer";
        case STQ_ERR_DEVICE: return "device error";
    }
    return "unknown status";
}

const char *stq_last_error(void) { return g_err.c_str(); }

stq_status stq_check_slot_ids(const stq_pool *pool, int32_t B, const int32_t *h_slot_ids) {
    g_err.clear();
    if (!pool || !pool->layout) return fail(STQ_ERR_INVALID, "pool is NULL");
    if (B < 0 || B > pool->slots) return fail(STQ_ERR_INVALID, "B must be in [0, slots]");
    if (B > 0 && !h_slot_ids) return fail(STQ_ERR_INVALID, "slot ids are NULL");
    return check_ids_host(pool->slots, B, h_slot_ids);
}

stq_status stq_pack_layout(const stq_config *cfg, stq_layout **out) {
    g_err.clear();
    if (!out) return fail(STQ_ERR_INVALID, "out is NULL");
    if (stq_status s = check_cfg(cfg)) return s;
    auto *L = new stq_layout;
    L->cfg = *cfg;
    L->cfg.unit_bits = nullptr;
    L->cfg.row_impact = nullptr;
    const bool keyrow = cfg->unit == STQ_UNIT_KEYROW;
    const int H = cfg->H, dk = cfg->d_k, dv = cfg->d_v, W = cfg->window, K = cfg->comps;
    L->bits.assign(cfg->unit_bits, cfg->unit_bits + (size_t)H * (keyrow ? dk : 1));
    L->heads.resize(H);
    L->rows.resize((size_t)H * dk);
    size_t slot = 0;
    size_t min_quant_entries = SIZE_MAX;
    for (int h = 0; h < H; ++h) {
        stq::HeadDesc d{};
        d.off = (uint32_t)slot;
        d.rows = (uint32_t)((size_t)h * dk);
        size_t p = 0;
        int nq = 0, common = -1;
        for (int i = 0; i < dk; ++i) {
            const int b = keyrow ? L->bits[(size_t)h * dk + i] : L->bits[h];
            L->rows[(size_t)h * dk + i] = stq::row_entry((uint32_t)p, (uint32_t)b);
            p += (size_t)dv * b / 8;
            nq += b < 16;
            common = (common == -1 || common == b) ? b : 0;
        }
        d.width = (uint16_t)common;
        d.nquant = (uint16_t)nq;
        if (common == 0) {
            L->mixed = true;
            bool w4p = true;
            for (int i = 0; i < dk; ++i) {
                const int b = keyrow ? L->bits[(size_t)h * dk + i] : L->bits[h];
                w4p &= b == 4 || b == 16;
            }
            if (w4p) {
                d.width = stq::kW4P;
                for (int i = 0; i < dk; ++i)
                    if (L->bits[(size_t)h * dk + i] == 16) d.pmask[i / 32] |= 1u << (i % 32);
            }
            L->step_mix = w4p ? (L->step_mix > 1 ? 2 : 1) : 2;
        }
        p = up(p, 16);
        if (nq > 0) {
            d.rs = (uint32_t)p;
            p = up(p + (size_t)dk * (cfg->row_scale == STQ_F16 ? 2 : 4), 16);
            if (cfg->col_scale == STQ_F16) {
                d.cs = (uint32_t)p;
                p = up(p + (size_t)dv * 2, 16);
            }
            if (cfg->scale_fit == STQ_FIT_LAGGED) {
                d.nrs = (uint32_t)p;
                p = up(p + (size_t)dk * (cfg->row_scale == STQ_F16 ? 2 : 4), 16);
                if (cfg->col_scale == STQ_F16) {
                    d.ncs = (uint32_t)p;
                    p = up(p + (size_t)dv * 2, 16);
                }
                d.srs = (uint32_t)p;
                p = up(p + (size_t)dk * 4, 16);
                if (cfg->col_scale == STQ_F16) {
                    d.scs = (uint32_t)p;
                    p = up(p + (size_t)dv * 4, 16);
                }
            }
        }
        if (W > 1) {
            d.wn = (uint32_t)p;   p = up(p + 4, 16);
            d.g = (uint32_t)p;    p = up(p + (size_t)dk * 4, 16);
            d.cidx = (uint32_t)p; p = up(p + (size_t)K * 2, 16);
            d.cval = (uint32_t)p; p = up(p + (size_t)K * 4, 16);
            d.du = (uint32_t)p;   p = up(p + (size_t)W * dv * 4, 16);
            d.dkap = (uint32_t)p; p = up(p + (size_t)W * dk * 4, 16);
        }
        d.bytes = (uint32_t)up(p, 256);
        slot += d.bytes;
        L->heads[h] = d;
        if ((size_t)nq * dv < min_quant_entries) min_quant_entries = (size_t)nq * dv;
    }
    if (W > 1 && (size_t)K > min_quant_entries) {
        delete L;
        return fail(STQ_ERR_INVALID, "comps exceeds the quantized entries of a head");
    }
    if (cfg->scale_fit == STQ_FIT_LAGGED && L->mixed) {
        delete L;
        return fail(STQ_ERR_UNSUPPORTED, "lagged scales need heads whose key rows share one width");
    }
    L->slot_bytes = slot;
    // Head groups of the step kernel: 4-bit heads in pairs (one workgroup
    // steps both, fetching the second while computing the first), every
    // other head alone.  The pairs come first: the grid runs group-major, so
    // a launch ends with the single heads, its shortest workgroups.
    std::vector<uint32_t> singles;
    int pending = -1;
    for (int h = 0; h < H; ++h) {
        if (L->heads[h].width != 4) {
            singles.push_back((uint32_t)h | 0xffff0000u);
        } else if (pending < 0) {
            pending = h;
        } else {
            L->groups.push_back((uint32_t)pending | ((uint32_t)h << 16));
            pending = -1;
        }
    }
    if (pending >= 0) singles.push_back((uint32_t)pending | 0xffff0000u);
    L->groups.insert(L->groups.end(), singles.begin(), singles.end());
    if (cfg->row_impact) {
        // w_i = sqrt(score_i / largest score of the head), in double, then fp32
        L->omega.assign((size_t)H * dk, 1.0f);
        for (int h = 0; h < H; ++h) {
            double mx = 0.0;
            for (int i = 0; i < dk; ++i) mx = std::fmax(mx, (double)cfg->row_impact[(size_t)h * dk + i]);
            if (mx > 0.0)
                for (int i = 0; i < dk; ++i)
                    L->omega[(size_t)h * dk + i] =
                        (float)std::sqrt((double)cfg->row_impact[(size_t)h * dk + i] / mx);
        }
    }
    const size_t hb = sizeof(stq::HeadDesc) * H, rb = sizeof(uint32_t) * (size_t)H * dk;
    const size_t gb = sizeof(uint32_t) * L->groups.size();
    const size_t ob = sizeof(float) * L->omega.size();
    // windowed layouts: an 8-byte window-end flag after the tables, 0 until a
    // call sets it (call tokens start at 1)
    L->flag_off = up(hb + rb + gb + ob, 8);
    const size_t fb = cfg->window > 1 ? 8 : 0;
    L->table.assign(up(L->flag_off + fb, 256), 0);
    std::memcpy(L->table.data(), L->heads.data(), hb);
    std::memcpy(L->table.data() + hb, L->rows.data(), rb);
    std::memcpy(L->table.data() + hb + rb, L->groups.data(), gb);
    if (ob) std::memcpy(L->table.data() + hb + rb + gb, L->omega.data(), ob);
    *out = L;
    return STQ_OK;
}

stq_status stq_layout_query(const stq_layout *L, size_t *slot_bytes, size_t *header_bytes) {
    g_err.clear();
    if (!L) return fail(STQ_ERR_INVALID, "layout is NULL");
    if (slot_bytes) *slot_bytes = L->slot_bytes;
    if (header_bytes) *header_bytes = L->table.size();
    return STQ_OK;
}

stq_status stq_layout_head(const stq_layout *L, int32_t h, size_t *offset, size_t *bytes) {
    g_err.clear();
    if (!L) return fail(STQ_ERR_INVALID, "layout is NULL");
    if (h < 0 || h >= L->cfg.H) return fail(STQ_ERR_INVALID, "head index out of range");
    if (offset) *offset = L->heads[h].off;
    if (bytes) *bytes = L->heads[h].bytes;
    return STQ_OK;
}

void stq_layout_free(stq_layout *L) { delete L; }

stq_status stq_alloc_pool(const stq_layout *L, int32_t slots, void *dev_base, size_t dev_bytes,
                          void *stream, stq_pool *out) {
    g_err.clear();
    if (!L || !out) return fail(STQ_ERR_INVALID, "layout or out is NULL");
    if (slots < 0) return fail(STQ_ERR_INVALID, "slots must be >= 0");
    const size_t need = L->table.size() + (size_t)slots * L->slot_bytes;
    if (!dev_base) {
        out->base = nullptr;
        out->bytes = need;
        out->slots = slots;
        out->layout = L;
        return STQ_OK;
    }
    if (!aligned(dev_base, 16)) return fail(STQ_ERR_ALIGN, "pool base must be 16-byte aligned");
    if (dev_bytes < need) return fail(STQ_ERR_TOO_SMALL, "pool buffer smaller than required");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(dev_base, L->table.data(), L->table.size(), hipMemcpyHostToDevice, s);
    if (stq_status st = launched(e, "table upload")) return st;
    uint8_t *slots_base = static_cast<uint8_t *>(dev_base) + L->table.size();
    e = stq::launch_pool_init(slots_base, L->slot_bytes, slots,
                              reinterpret_cast<const stq::HeadDesc *>(dev_base), L->cfg.H,
                              L->cfg.d_k, L->cfg.window, s);
    if (stq_status st = launched(e, "pool init")) return st;
    out->base = dev_base;
    out->bytes = need;
    out->slots = slots;
    out->layout = L;
    return STQ_OK;
}

stq_status stq_decode_step(const stq_pool *pool, int32_t B, const int32_t *d_slot_ids,
                           const void *d_q, const void *d_k, const void *d_v, const float *d_a,
                           const float *d_beta, float *d_o, void *stream) {
    g_err.clear();
    if (stq_status s = check_batch(pool, B, d_slot_ids)) return s;
    if (B == 0) return STQ_OK;
    const void *ptrs[] = {d_q, d_k, d_v, d_a, d_beta, d_o};
    for (const void *p : ptrs) {
        if (!p) return fail(STQ_ERR_INVALID, "an input or output pointer is NULL");
        if (!aligned(p, 16)) return fail(STQ_ERR_ALIGN, "device pointers must be 16-byte aligned");
    }
    const stq_layout *L = pool->layout;
    stq::Args a = base_args(pool, B, d_slot_ids);
    a.q = d_q;
    a.k = d_k;
    a.v = d_v;
    a.a = d_a;
    a.beta = d_beta;
    a.o = d_o;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (L->cfg.window > 1) {
        a.token = g_token.fetch_add(1, std::memory_order_relaxed) + 1;
        return launched(stq::launch_step_win(a, L->cfg.d_k, L->cfg.d_v, L->mixed, s), "windowed decode step");
    }
    if (L->cfg.scale_fit == STQ_FIT_LAGGED)
        return launched(stq::launch_step_lagged(a, L->cfg.d_k, L->cfg.d_v, s), "decode step (lagged scales)");
    return launched(stq::launch_step(a, L->cfg.d_k, L->cfg.d_v, L->step_mix, s), "decode step");
}

stq_status stq_fit_scales(const stq_pool *pool, int32_t B, const int32_t *d_slot_ids, void *stream) {
    g_err.clear();
    if (stq_status s = check_batch(pool, B, d_slot_ids)) return s;
    const stq_layout *L = pool->layout;
    if (L->cfg.scale_fit != STQ_FIT_LAGGED)
        return fail(STQ_ERR_INVALID, "the layout has no lagged scales (scale_fit is STQ_FIT_STEP)");
    if (B == 0) return STQ_OK;
    stq::Args a = base_args(pool, B, d_slot_ids);
    return launched(stq::launch_fit(a, L->cfg.d_k, L->cfg.d_v, static_cast<hipStream_t>(stream)), "scale fit");
}

stq_status stq_unpack(const stq_pool *pool, int32_t B, const int32_t *d_slot_ids, float *d_state,
                      void *stream) {
    g_err.clear();
    if (stq_status s = check_batch(pool, B, d_slot_ids)) return s;
    if (B == 0) return STQ_OK;
    if (!d_state) return fail(STQ_ERR_INVALID, "state pointer is NULL");
    if (!aligned(d_state, 16)) return fail(STQ_ERR_ALIGN, "state must be 16-byte aligned");
    const stq_layout *L = pool->layout;
    stq::Args a = base_args(pool, B, d_slot_ids);
    a.state = d_state;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (L->cfg.window > 1) return launched(stq::launch_unpack_win(a, L->cfg.d_k, L->cfg.d_v, s), "unpack");
    return launched(stq::launch_unpack(a, L->cfg.d_k, L->cfg.d_v, s), "unpack");
}

stq_status stq_pack(const stq_pool *pool, int32_t B, const int32_t *d_slot_ids,
                    const float *d_state, void *stream) {
    g_err.clear();
    if (stq_status s = check_batch(pool, B, d_slot_ids)) return s;
    if (B == 0) return STQ_OK;
    if (!d_state) return fail(STQ_ERR_INVALID, "state pointer is NULL");
    if (!aligned(d_state, 16)) return fail(STQ_ERR_ALIGN, "state must be 16-byte aligned");
    const stq_layout *L = pool->layout;
    stq::Args a = base_args(pool, B, d_slot_ids);
    a.state = const_cast<float *>(d_state);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (L->cfg.window > 1)
        return launched(stq::launch_pack_win(a, L->cfg.d_k, L->cfg.d_v, L->mixed, s), "pack");
    return launched(stq::launch_pack(a, L->cfg.d_k, L->cfg.d_v, s), "pack");
}

}  // extern "C"
