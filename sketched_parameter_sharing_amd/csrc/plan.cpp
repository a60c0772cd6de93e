// Host-side plan of an SS1 layer: the seeded balanced chunk hash with +-1
// signs for every neuron group, its validation and its inverse index.
//
// The pages fix only that SS1's parameter sharing is random, confined to each
// neuron's weight vector and coalesced along K and N ("SS1: Accelerating
// Inference with Fast and Expressive Sketch Structured Transform", summary
// page, "Approach").  How the randomness is drawn is this library's own
// choice, documented with ss1_plan in ss1.h.
#include "ss1_internal.h"

#include <vector>

namespace ss1 {

namespace {

// SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): a Weyl sequence with the
// golden-ratio increment, each state passed through a 64-bit finaliser.
struct SplitMix64 {
    uint64_t state;
    explicit SplitMix64(uint64_t seed) : state(seed) {}
    uint64_t next() {
        state += 0x9E3779B97F4A7C15ull;
        uint64_t z = state;
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
};

}  // namespace

ss1_status check_chunking(int64_t K, int64_t N, int32_t c, int32_t BK, int32_t BN, Dims* d) {
    if (K <= 0 || N <= 0 || c <= 0 || BK <= 0 || BN <= 0) return SS1_ERR_SHAPE;
    if (c > SS1_MAX_C) return SS1_ERR_SHAPE;
    if (K % BK != 0) return SS1_ERR_SHAPE;
    const int64_t J = K / BK;
    if (J % c != 0) return SS1_ERR_SHAPE;
    if (J > SS1_MAX_CHUNKS) return SS1_ERR_SHAPE;
    if (N % BN != 0) return SS1_ERR_SHAPE;
    if (d) {
        d->K = K;
        d->N = N;
        d->c = c;
        d->BK = BK;
        d->BN = BN;
        d->J = J;
        d->Jc = J / c;
        d->Kc = K / c;
        d->G = N / BN;
    }
    return SS1_OK;
}

}  // namespace ss1

using ss1::Dims;

extern "C" ss1_status ss1_plan(uint64_t seed, int64_t K, int64_t N, int32_t c, int32_t BK,
                               int32_t BN, int32_t* hash, int8_t* sign) {
    Dims d;
    ss1_status st = ss1::check_chunking(K, N, c, BK, BN, &d);
    if (st != SS1_OK) return st;
    if (!hash || !sign) return SS1_ERR_NULL;
    ss1::SplitMix64 rng(seed);
    std::vector<int32_t> order(static_cast<size_t>(d.J));
    for (int64_t g = 0; g < d.G; ++g) {
        for (int64_t j = 0; j < d.J; ++j) order[j] = static_cast<int32_t>(j);
        for (int64_t i = d.J - 1; i >= 1; --i) {
            const uint64_t k = rng.next() % static_cast<uint64_t>(i + 1);
            const int32_t tmp = order[i];
            order[i] = order[k];
            order[k] = tmp;
        }
        int32_t* hg = hash + g * d.J;
        int8_t* sg = sign + g * d.J;
        for (int64_t p = 0; p < d.J; ++p) hg[order[p]] = static_cast<int32_t>(p / c);
        for (int64_t j = 0; j < d.J; ++j) sg[j] = (rng.next() >> 63) ? int8_t(-1) : int8_t(1);
    }
    return SS1_OK;
}

extern "C" ss1_status ss1_plan_index(const int32_t* hash, const int8_t* sign, int64_t K, int64_t N,
                                     int32_t c, int32_t BK, int32_t BN, int32_t* idx,
                                     int8_t* isign) {
    Dims d;
    ss1_status st = ss1::check_chunking(K, N, c, BK, BN, &d);
    if (st != SS1_OK) return st;
    if (!hash || !sign || !idx || !isign) return SS1_ERR_NULL;
    std::vector<int32_t> fill(static_cast<size_t>(d.Jc));
    for (int64_t g = 0; g < d.G; ++g) {
        const int32_t* hg = hash + g * d.J;
        const int8_t* sg = sign + g * d.J;
        int32_t* ig = idx + g * d.Jc * c;
        int8_t* isg = isign + g * d.Jc * c;
        for (int64_t t = 0; t < d.Jc; ++t) fill[t] = 0;
        // ascending j fills each compressed chunk's sources in ascending order
        for (int64_t j = 0; j < d.J; ++j) {
            const int32_t t = hg[j];
            if (t < 0 || t >= d.Jc) return SS1_ERR_PLAN;
            if (sg[j] != 1 && sg[j] != -1) return SS1_ERR_PLAN;
            if (fill[t] >= c) return SS1_ERR_PLAN;
            ig[t * c + fill[t]] = static_cast<int32_t>(j);
            isg[t * c + fill[t]] = sg[j];
            ++fill[t];
        }
        for (int64_t t = 0; t < d.Jc; ++t)
            if (fill[t] != c) return SS1_ERR_PLAN;
    }
    return SS1_OK;
}
