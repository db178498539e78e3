// Host-only driver of the library's allocator and prefix cache (allocator.cpp,
// sha256.cpp), built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py.  It reads one command per line on stdin, calls the
// C ABI and prints what came back, so the test can compare every answer with the
// oracle's allocator while the sanitizers watch every access.
//
// Commands (integers separated by blanks):
//   P nb bs flags n order[n]     create a host-only pool (n = 0: identity order)
//   C                             seq_create           -> "C st id"
//   F parent                      seq_fork             -> "F st id"
//   A seq n                       seq_append           -> "A st slots... / copies..."
//   K seq n tok[n]                seq_append_tokens    -> "K st slots... / copies..."
//   Q n extra tok[n]              seq_create_prefix    -> "Q st id n_cached"
//   B k seq[k] count[k]           append_batch         -> "B st n_done slots... / copies..."
//   X seq                         seq_free             -> "X st"
//   T k width seq[k]              block_tables         -> "T st len table[width] ..."
//   S                             stats + prefix stats -> "S free used waste cached hits ev"
//   R                             every block's count  -> "R c0 c1 ..."
//   E                             invalid-argument probes -> "E ok" or "E fail <what>"
//   D                             destroy the pool
#include <cstdint>
#include <cstdio>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "paged_kv.h"

static paged_kv_pool* g_pool = nullptr;
static paged_kv_pool_desc g_desc{};

static void print_lists(const std::vector<int32_t>& a, const std::vector<int32_t>& b) {
    for (int32_t x : a) std::printf(" %d", x);
    std::printf(" /");
    for (int32_t x : b) std::printf(" %d", x);
    std::printf("\n");
}

static std::vector<int32_t> read_n(std::istringstream& in, int64_t n) {
    std::vector<int32_t> v((size_t)n);
    for (auto& x : v) in >> x;
    return v;
}

static bool probes() {
    // every call here must fail cleanly, never touch memory it was not given
    paged_kv_pool* p = nullptr;
    paged_kv_pool_desc bad = g_desc;
    bad.num_blocks = 0;
    if (paged_kv_pool_create(&bad, nullptr, nullptr, nullptr, &p) != PAGED_KV_ERR_INVALID_ARG || p) return false;
    bad = g_desc;
    bad.flags = PAGED_KV_POOL_HOST_ONLY;
    std::vector<int32_t> dup(g_desc.num_blocks, 0);   // not a permutation
    if (g_desc.num_blocks > 1 &&
        paged_kv_pool_create(&bad, dup.data(), nullptr, nullptr, &p) != PAGED_KV_ERR_INVALID_ARG) return false;
    int32_t id = 0, nc = 0;
    int32_t slots[4], copies[2];
    if (paged_kv_seq_append(g_pool, -1, 1, slots, copies, 1, &nc) != PAGED_KV_ERR_NO_SUCH_SEQ) return false;
    if (paged_kv_seq_append(g_pool, 1 << 30, 1, slots, copies, 1, &nc) != PAGED_KV_ERR_NO_SUCH_SEQ) return false;
    if (paged_kv_seq_fork(g_pool, 1 << 30, &id) != PAGED_KV_ERR_NO_SUCH_SEQ) return false;
    if (paged_kv_seq_free(g_pool, -5) != PAGED_KV_ERR_NO_SUCH_SEQ) return false;
    int32_t rc = 0;
    if (paged_kv_block_refcount(g_pool, -1, &rc) == PAGED_KV_OK) return false;
    if (paged_kv_block_refcount(g_pool, g_desc.num_blocks, &rc) == PAGED_KV_OK) return false;
    if (paged_kv_block_hash(nullptr, nullptr, 3, 0, nullptr) == PAGED_KV_OK) return false;
    uint8_t out[32];
    if (paged_kv_block_hash(nullptr, nullptr, 0, 7, out) != PAGED_KV_OK) return false;
    if (paged_kv_pool_bytes(nullptr) != 0) return false;
    if (paged_kv_bytes_per_token(80, 8, 128, 2) != 327680ull) return false;
    if (paged_kv_status_string((paged_kv_status)99) == nullptr) return false;
    return true;
}

int main() {
    std::string line;
    while (std::getline(std::cin, line)) {
        std::istringstream in(line);
        char c = 0;
        if (!(in >> c)) continue;
        if (c == 'P') {
            int64_t nb, bs, flags, n;
            in >> nb >> bs >> flags >> n;
            std::vector<int32_t> order = read_n(in, n);
            g_desc = paged_kv_pool_desc{(int32_t)nb, (int32_t)bs, 1, 64, PAGED_KV_BF16,
                                        (int32_t)(flags | PAGED_KV_POOL_HOST_ONLY)};
            int st = paged_kv_pool_create(&g_desc, n ? order.data() : nullptr, nullptr, nullptr, &g_pool);
            std::printf("P %d\n", st);
        } else if (c == 'C') {
            int32_t id = -1;
            int st = paged_kv_seq_create(g_pool, &id);
            std::printf("C %d %d\n", st, id);
        } else if (c == 'F') {
            int32_t parent, id = -1;
            in >> parent;
            int st = paged_kv_seq_fork(g_pool, parent, &id);
            std::printf("F %d %d\n", st, id);
        } else if (c == 'A' || c == 'K') {
            int32_t seq, n;
            in >> seq >> n;
            std::vector<int32_t> toks = c == 'K' ? read_n(in, n) : std::vector<int32_t>();
            std::vector<int32_t> slots((size_t)n + 1), copies(2);
            int32_t nc = 0;
            int st = c == 'K' ? paged_kv_seq_append_tokens(g_pool, seq, toks.data(), n, slots.data(),
                                                           copies.data(), 1, &nc)
                              : paged_kv_seq_append(g_pool, seq, n, slots.data(), copies.data(), 1, &nc);
            slots.resize(st == PAGED_KV_OK ? (size_t)n : 0);
            copies.resize(st == PAGED_KV_OK ? 2 * (size_t)nc : 0);
            std::printf("%c %d", c, st);
            print_lists(slots, copies);
        } else if (c == 'Q') {
            int32_t n;
            int64_t extra;
            in >> n >> extra;
            std::vector<int32_t> toks = read_n(in, n);
            int32_t id = -1, nc = -1;
            int st = paged_kv_seq_create_prefix(g_pool, toks.data(), n, extra, &id, &nc);
            std::printf("Q %d %d %d\n", st, id, nc);
        } else if (c == 'B') {
            int32_t k;
            in >> k;
            std::vector<int32_t> seqs = read_n(in, k), counts = read_n(in, k);
            int64_t total = 0;
            for (int32_t x : counts) total += x;
            std::vector<int32_t> slots((size_t)total + 1), copies(2 * (size_t)k + 2);
            int32_t nc = 0, nd = 0;
            int st = paged_kv_append_batch(g_pool, seqs.data(), counts.data(), k, slots.data(),
                                           copies.data(), k + 1, &nc, &nd);
            int64_t written = 0;
            for (int32_t i = 0; i < nd; ++i) written += counts[i];
            slots.resize(st == PAGED_KV_OK ? (size_t)written : 0);
            copies.resize(st == PAGED_KV_OK ? 2 * (size_t)nc : 0);
            std::printf("B %d %d", st, nd);
            print_lists(slots, copies);
        } else if (c == 'X') {
            int32_t seq;
            in >> seq;
            std::printf("X %d\n", paged_kv_seq_free(g_pool, seq));
        } else if (c == 'T') {
            int32_t k, width;
            in >> k >> width;
            std::vector<int32_t> seqs = read_n(in, k);
            std::vector<int32_t> tables((size_t)k * width), lens(k);
            int st = paged_kv_block_tables(g_pool, seqs.data(), k, width, tables.data(), lens.data());
            std::printf("T %d", st);
            if (st == PAGED_KV_OK)
                for (int32_t i = 0; i < k; ++i) {
                    std::printf(" %d :", lens[i]);
                    for (int32_t j = 0; j < width; ++j) std::printf(" %d", tables[(size_t)i * width + j]);
                    std::printf(" ;");
                }
            std::printf("\n");
        } else if (c == 'S') {
            int64_t f = 0, u = 0, w = 0, ca = 0, h = 0, e = 0;
            paged_kv_stats(g_pool, &f, &u, &w);
            if (g_desc.flags & PAGED_KV_POOL_PREFIX_CACHE) paged_kv_prefix_stats(g_pool, &ca, &h, &e);
            std::printf("S %lld %lld %lld %lld %lld %lld\n", (long long)f, (long long)u, (long long)w,
                        (long long)ca, (long long)h, (long long)e);
        } else if (c == 'R') {
            std::printf("R");
            for (int32_t b = 0; b < g_desc.num_blocks; ++b) {
                int32_t rc = -1;
                paged_kv_block_refcount(g_pool, b, &rc);
                std::printf(" %d", rc);
            }
            std::printf("\n");
        } else if (c == 'E') {
            std::printf("E %s\n", probes() ? "ok" : "fail");
        } else if (c == 'D') {
            paged_kv_pool_destroy(g_pool);
            g_pool = nullptr;
        }
    }
    if (g_pool) paged_kv_pool_destroy(g_pool);
    return 0;
}
