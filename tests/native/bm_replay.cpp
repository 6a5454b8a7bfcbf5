// Replays a block-manager trace through libpa's C++ block manager, for the
// sanitizer test (tests/test_block_manager_sanitized.py builds this file
// together with the manager's source under AddressSanitizer and
// UndefinedBehaviorSanitizer and compares what it prints with the reference
// model's results).  Test infrastructure, not part of the library.
//
// Input, one command per line (integers separated by spaces):
//   create N B prefix_cache k order_0 .. order_{k-1}   device manager (k = 0: identity order)
//   host N B                                           host manager for swaps
//   add S L p_0 .. p_{L-1}                ->  rc cached
//   append S n k t_0 .. t_{k-1}           ->  rc n_slots slots.. n_pairs src dst ..
//   batch m s_0 .. s_{m-1} k t_0 ..       ->  rc done n_slots slots.. n_pairs src dst ..
//   fork P C                              ->  rc
//   free S                                ->  rc
//   swapout S / swapin S                  ->  rc n_pairs src dst ..
//   state m s_0 .. s_{m-1}                ->  num_free num_cached host_free
//                                             (len blocks b..) per sequence, then every ref count
// Each command's result is one output line.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "pa.h"
#include "pa_block_manager.h"

namespace {

std::vector<int64_t> read_ints(std::istringstream& in, int64_t n) {
    std::vector<int64_t> v(static_cast<size_t>(n));
    for (auto& x : v) in >> x;
    return v;
}

std::vector<int32_t> to32(const std::vector<int64_t>& v) { return std::vector<int32_t>(v.begin(), v.end()); }

void print_pairs(std::ostringstream& out, const std::vector<int64_t>& pairs, int32_t n) {
    out << ' ' << n;
    for (int32_t i = 0; i < 2 * n; ++i) out << ' ' << pairs[static_cast<size_t>(i)];
}

}  // namespace

int main() {
    pa_bm* bm = nullptr;
    pa_bm* host = nullptr;
    int64_t num_blocks = 0, host_blocks = 0;
    int32_t block_size = 1;
    std::string line;
    while (std::getline(std::cin, line)) {
        std::istringstream in(line);
        std::string cmd;
        in >> cmd;
        std::ostringstream out;
        if (cmd == "create") {
            int64_t n, b, pc, k;
            in >> n >> b >> pc >> k;
            const std::vector<int32_t> order = to32(read_ints(in, k));
            bm = pa_bm_create(n, static_cast<int32_t>(b), k ? order.data() : nullptr, static_cast<int32_t>(pc));
            num_blocks = n;
            block_size = static_cast<int32_t>(b);
            out << (bm ? 0 : 1);
        } else if (cmd == "host") {
            int64_t n, b;
            in >> n >> b;
            host = pa_bm_create(n, static_cast<int32_t>(b), nullptr, 0);
            host_blocks = n;
            out << (host ? 0 : 1);
        } else if (cmd == "add") {
            int64_t s, l;
            in >> s >> l;
            const std::vector<int32_t> prompt = to32(read_ints(in, l));
            int32_t cached = -1;
            const int rc = pa_bm_add_seq(bm, s, l ? prompt.data() : nullptr, static_cast<int32_t>(l), &cached);
            out << rc << ' ' << cached;
        } else if (cmd == "append") {
            int64_t s, n, k;
            in >> s >> n >> k;
            const std::vector<int32_t> toks = to32(read_ints(in, k));
            std::vector<int64_t> slots(static_cast<size_t>(n > 0 ? n : 1)), pair(2, -1);
            int32_t np = 0;
            const int rc = pa_bm_append(bm, s, static_cast<int32_t>(n), k ? toks.data() : nullptr, slots.data(),
                                        pair.data(), &np);
            out << rc << ' ' << (rc == PA_OK ? n : 0);
            if (rc == PA_OK)
                for (int64_t i = 0; i < n; ++i) out << ' ' << slots[static_cast<size_t>(i)];
            print_pairs(out, pair, rc == PA_OK ? np : 0);
        } else if (cmd == "batch") {
            int64_t m;
            in >> m;
            const std::vector<int64_t> seqs = read_ints(in, m);
            int64_t k;
            in >> k;
            const std::vector<int32_t> toks = to32(read_ints(in, k));
            std::vector<int64_t> slots(static_cast<size_t>(m)), pairs(static_cast<size_t>(2 * m), -1);
            int32_t np = 0, done = -1;
            const int rc = pa_bm_append_batch(bm, seqs.data(), static_cast<int32_t>(m), k ? toks.data() : nullptr,
                                              slots.data(), pairs.data(), &np, &done);
            const int64_t ns = rc == PA_OK ? m : done;
            out << rc << ' ' << done << ' ' << ns;
            for (int64_t i = 0; i < ns; ++i) out << ' ' << slots[static_cast<size_t>(i)];
            print_pairs(out, pairs, np);
        } else if (cmd == "fork") {
            int64_t p, c;
            in >> p >> c;
            out << pa_bm_fork(bm, p, c);
        } else if (cmd == "free") {
            int64_t s;
            in >> s;
            out << pa_bm_free_seq(bm, s);
        } else if (cmd == "swapout" || cmd == "swapin") {
            int64_t s;
            in >> s;
            const int64_t cap = std::max(num_blocks, host_blocks);
            std::vector<int64_t> pairs(static_cast<size_t>(2 * cap), -1);
            int32_t np = 0;
            const int rc = cmd == "swapout"
                               ? pa_bm_swap_out(bm, host, s, pairs.data(), static_cast<int32_t>(cap), &np)
                               : pa_bm_swap_in(bm, host, s, pairs.data(), static_cast<int32_t>(cap), &np);
            out << rc;
            print_pairs(out, pairs, rc == PA_OK ? np : 0);
        } else if (cmd == "state") {
            int64_t m;
            in >> m;
            const std::vector<int64_t> seqs = read_ints(in, m);
            out << pa_bm_num_free(bm) << ' ' << pa_bm_num_cached(bm) << ' ' << pa_bm_num_free(host);
            const int32_t width = static_cast<int32_t>((num_blocks > 0 ? num_blocks : 1));
            std::vector<int32_t> tables(static_cast<size_t>(width * (m > 0 ? m : 1))), lens(static_cast<size_t>(m > 0 ? m : 1));
            if (m > 0) {
                const int rc = pa_bm_block_tables(bm, seqs.data(), static_cast<int32_t>(m), width, tables.data(),
                                                  lens.data());
                if (rc != PA_OK) {
                    std::printf("block_tables failed: %d\n", rc);
                    return 2;
                }
            }
            for (int64_t i = 0; i < m; ++i) {
                const int32_t held = pa_bm_num_blocks_held(bm, seqs[static_cast<size_t>(i)]);
                out << " | " << lens[static_cast<size_t>(i)] << ' ' << held;
                for (int32_t j = 0; j < held; ++j) out << ' ' << tables[static_cast<size_t>(i * width + j)];
            }
            out << " |";
            for (int64_t b = 0; b < num_blocks; ++b) out << ' ' << pa_bm_ref_count(bm, static_cast<int32_t>(b));
        } else if (cmd.empty()) {
            continue;
        } else {
            std::printf("unknown command %s\n", cmd.c_str());
            return 2;
        }
        std::printf("%s\n", out.str().c_str());
    }
    (void)block_size;
    pa_bm_destroy(host);
    pa_bm_destroy(bm);
    return 0;
}
