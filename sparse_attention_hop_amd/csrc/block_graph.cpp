// Host construction of two static layouts, as CSR graphs for import
// ("1.2.1 Static sparsity": section 2, eq. 13, the BigBird block graph;
// section 1.2, eqs. 11 and 12, Longformer's dilated window with globals).
#include <algorithm>
#include <cstdint>
#include <vector>

#include "internal.h"

namespace diffuser {
namespace {

// SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): output function and the
// counter-th output of a generator seeded with `seed`.
uint64_t splitmix_mix_host(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

uint64_t splitmix_at(uint64_t seed, uint64_t counter) {
    return splitmix_mix_host(seed + 0x9E3779B97F4A7C15ull * (counter + 1ull));
}

}  // namespace

bool build_block_lists(int64_t nblocks, int32_t local_blocks, int32_t num_random,
                       int32_t num_global, int32_t num_graphs, uint64_t seed,
                       std::vector<std::vector<int32_t>>& keys) {
    const int64_t N = nblocks, h = (local_blocks - 1) / 2;
    keys.assign((size_t)num_graphs * N, {});
    std::vector<char> mark((size_t)N);
    for (int64_t gr = 0; gr < num_graphs; ++gr) {
        for (int64_t I = 0; I < N; ++I) {
            std::vector<int32_t>& ks = keys[(size_t)(gr * N + I)];
            if (I < num_global) {
                ks.resize((size_t)N);
                for (int64_t J = 0; J < N; ++J) ks[(size_t)J] = (int32_t)J;
                continue;
            }
            std::fill(mark.begin(), mark.end(), 0);
            int64_t taken = 0;
            for (int64_t J = std::max<int64_t>(0, I - h); J <= std::min<int64_t>(N - 1, I + h); ++J)
                if (!mark[(size_t)J]) mark[(size_t)J] = 1, ++taken;
            for (int64_t J = 0; J < num_global; ++J)
                if (!mark[(size_t)J]) mark[(size_t)J] = 1, ++taken;
            const int64_t pool = N - taken;
            if (pool <= num_random) {
                std::fill(mark.begin(), mark.end(), 1);
            } else {
                const uint64_t row = ((uint64_t)(gr * N + I)) << 20;
                int64_t got = 0;
                for (uint64_t t = 0; got < num_random; ++t) {
                    if (t >= (1ull << 20)) return false;
                    const uint64_t u = splitmix_at(seed, row | t);
                    const int64_t J = (int64_t)(((u >> 32) * (uint64_t)N) >> 32);
                    if (!mark[(size_t)J]) mark[(size_t)J] = 2, ++got;
                }
            }
            for (int64_t J = 0; J < N; ++J)
                if (mark[(size_t)J]) ks.push_back((int32_t)J);
        }
    }
    return true;
}

void block_lists_to_csr(int64_t n, int32_t block, int32_t num_graphs,
                        const std::vector<std::vector<int32_t>>& keys,
                        std::vector<int64_t>& row_ptr, std::vector<int32_t>& cols) {
    const int64_t N = n / block;
    row_ptr.assign((size_t)num_graphs * (n + 1), 0);
    cols.clear();
    for (int64_t gr = 0; gr < num_graphs; ++gr) {
        int64_t* rp = row_ptr.data() + gr * (n + 1);
        for (int64_t i = 0; i < n; ++i) {
            const std::vector<int32_t>& ks = keys[(size_t)(gr * N + i / block)];
            for (int32_t J : ks)
                for (int32_t c = 0; c < block; ++c) cols.push_back(J * block + c);
            rp[i + 1] = rp[i] + (int64_t)ks.size() * block;
        }
    }
}

void dilated_csr(int64_t n, int32_t radius, int32_t dilation, const int32_t* G, int32_t g,
                 std::vector<int64_t>& row_ptr, std::vector<int32_t>& cols) {
    std::vector<char> is_global((size_t)n, 0);
    for (int32_t q = 0; q < g; ++q) is_global[(size_t)G[q]] = 1;
    row_ptr.assign((size_t)n + 1, 0);
    cols.clear();
    std::vector<int32_t> row;
    for (int64_t i = 0; i < n; ++i) {
        row.clear();
        if (is_global[(size_t)i]) {
            for (int64_t j = 0; j < n; ++j) row.push_back((int32_t)j);
        } else {
            for (int64_t k = -radius; k <= radius; ++k) {
                const int64_t j = i + k * (int64_t)dilation;
                if (j >= 0 && j < n) row.push_back((int32_t)j);
            }
            for (int32_t q = 0; q < g; ++q) row.push_back(G[q]);
            std::sort(row.begin(), row.end());
            row.erase(std::unique(row.begin(), row.end()), row.end());
        }
        cols.insert(cols.end(), row.begin(), row.end());
        row_ptr[(size_t)i + 1] = (int64_t)cols.size();
    }
}

}  // namespace diffuser
