// Lifetime-aware bit allocation (host only): the unit widths a layout takes.
//
// STEPQuant essay, temporal-axis paragraphs and the Proposition 1 discussion:
// an error the update does not remove fades only by the gate, so an error in a
// unit with mean gate a persists for about 1 / (1 - a) steps; within a fixed
// average width, bits go to the units whose error is both large and long-lived,
// and the riskiest few stay FP16 pivots.  Reading used (the pages give no
// formula): weight s_u = m_u / (1 - min(a_u, 1 - 2^-20)) with m_u the unit's
// mean squared state entry; the n_pivots largest weights become pivots; every
// other unit starts at 4 bits and, while 2 more bits fit in
// floor(avg_bits * others), the unit with the largest risk reduction
// s_u * (4^-b - 4^-(b+2)) = s_u * 15 * 2^-(2b+4) moves up one width (ties: lower
// unit index).  All arithmetic is in double, in that order.
#include <cmath>
#include <cstdint>
#include <queue>
#include <string>
#include <vector>

#include "stq.h"

namespace stq {
void set_error(const std::string &msg);
}

namespace {

struct Cand {
    double gain;
    int32_t unit;
};
// max-heap on gain, then on the lower unit index
struct Lower {
    bool operator()(const Cand &x, const Cand &y) const {
        if (x.gain != y.gain) return x.gain < y.gain;
        return x.unit > y.unit;
    }
};

double weight(float a, float m) {
    const double cap = 1.0 - std::ldexp(1.0, -20);
    const double ad = (double)a < cap ? (double)a : cap;
    const double life = 1.0 / (1.0 - ad);
    return life * (double)m;
}

double gain(double s, int b) { return s * (15.0 * std::ldexp(1.0, -(2 * b + 4))); }

}  // namespace

extern "C" stq_status stq_allocate_bits(int32_t n_units, const float *gate_mean, const float *state_msq,
                                        double avg_bits, int32_t n_pivots, uint8_t *unit_bits) {
    stq::set_error("");
    if (n_units < 1 || !gate_mean || !state_msq || !unit_bits) {
        stq::set_error("n_units must be >= 1 and the arrays non-NULL");
        return STQ_ERR_INVALID;
    }
    if (!(avg_bits >= 4.0 && avg_bits <= 8.0)) {
        stq::set_error("avg_bits must be in [4, 8]");
        return STQ_ERR_INVALID;
    }
    if (n_pivots < 0 || n_pivots > n_units) {
        stq::set_error("n_pivots must be in [0, n_units]");
        return STQ_ERR_INVALID;
    }
    std::vector<double> s((size_t)n_units);
    for (int32_t u = 0; u < n_units; ++u) {
        const float a = gate_mean[u], m = state_msq[u];
        if (!(a >= 0.0f && a <= 1.0f) || !(m >= 0.0f) || !std::isfinite(m)) {
            stq::set_error("gate means must be in [0, 1] and mean squares finite and >= 0");
            return STQ_ERR_INVALID;
        }
        s[(size_t)u] = weight(a, m);
    }
    std::vector<uint8_t> bits((size_t)n_units, 4);
    // pivots: the n_pivots largest weights (lower index first among equals)
    std::priority_queue<Cand, std::vector<Cand>, Lower> piv;
    for (int32_t u = 0; u < n_units; ++u) piv.push({s[(size_t)u], u});
    for (int32_t p = 0; p < n_pivots; ++p) {
        bits[(size_t)piv.top().unit] = 16;
        piv.pop();
    }
    const int64_t others = n_units - n_pivots;
    const int64_t budget = (int64_t)std::floor(avg_bits * (double)others);
    int64_t used = 4 * others;
    std::priority_queue<Cand, std::vector<Cand>, Lower> up;
    for (int32_t u = 0; u < n_units; ++u)
        if (bits[(size_t)u] != 16) up.push({gain(s[(size_t)u], 4), u});
    while (!up.empty() && used + 2 <= budget) {
        const int32_t u = up.top().unit;
        up.pop();
        bits[(size_t)u] = (uint8_t)(bits[(size_t)u] + 2);
        used += 2;
        if (bits[(size_t)u] < 8) up.push({gain(s[(size_t)u], bits[(size_t)u]), u});
    }
    for (int32_t u = 0; u < n_units; ++u) unit_bits[u] = bits[(size_t)u];
    return STQ_OK;
}
