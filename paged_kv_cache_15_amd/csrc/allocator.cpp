// Host block allocator of the paged KV cache and the pool object behind the C ABI.
//
// What it implements (deepsonar "PagedAttention de vLLM …"):
//   §2.2  fixed-size physical blocks, a per-sequence table from logical to physical
//         block, a new block only once the previous one is full;
//   §2.3  reference counts on shared blocks, copy before writing into a shared one;
//   §2.4  a FIFO free-block queue: allocation pops the head, release pushes the tail.
// deeplearn.tn "PagedAttention : comment optimiser la mémoire GPU …", worked example:
// the token that overflows a full block lands at offset 0 of a newly taken block.
//
// With PAGED_KV_POOL_PREFIX_CACHE (§2.4, hash chain of V1; §VII step 5): every full
// block written through paged_kv_seq_append_tokens gets a chained hash,
// SHA-256(parent block's hash, its token ids, an extra key); a map from hash to block
// lets a new prompt take over the cached blocks its chain matches (all but the last
// prompt token, which is always recomputed); released blocks keep their hash while
// they wait in the free queue, and a cached block is evicted from the map when
// allocation takes it from the queue head, so the queue order is the LRU order.
//
// Readings where the pages are silent: the initial queue order is caller input;
// released blocks go back in logical order; a copy-on-write copies a whole block and
// the last holder writes in place; a failed append changes nothing; sequence ids are
// sequential and never reused.  Hash input: parent digest (32 zero bytes for the first
// block), token ids as little-endian int32, extra key as little-endian int64; only full
// blocks are hashed; a hash already in the map keeps its older block; a matched block
// waiting in the free queue leaves the queue; a sequence appended to without token ids
// registers no blocks.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cstdarg>
#include <cstring>
#include <unordered_map>
#include <vector>

#include "common.h"
#include "sha256.h"

namespace pkv {

static thread_local std::string g_last_error;

void set_error(const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
}

void clear_error() { g_last_error.clear(); }

bool valid_desc(const paged_kv_pool_desc* d) {
    if (!d) { set_error("null pool descriptor"); return false; }
    if (d->num_blocks < 1 || d->block_size < 1 || d->num_kv_heads < 1 || d->head_dim < 1) {
        set_error("pool sizes must be >= 1 (blocks %d, block_size %d, kv_heads %d, head_dim %d)",
                  d->num_blocks, d->block_size, d->num_kv_heads, d->head_dim);
        return false;
    }
    int eb = elem_bytes(d->dtype);
    if (!eb) { set_error("unknown dtype %d", d->dtype); return false; }
    if ((d->head_dim * eb) % 16) {
        set_error("head_dim %d is not a multiple of the 16-byte chunk", d->head_dim);
        return false;
    }
    if ((int64_t)d->num_blocks * d->block_size > INT32_MAX) {
        set_error("num_blocks * block_size does not fit an int32 slot id");
        return false;
    }
    return true;
}

bool kernel_desc(const paged_kv_pool_desc* d, bool attention) {
    if (!valid_desc(d)) return false;
    if (d->block_size != 1 && d->block_size != 16 && d->block_size != 32) {
        set_error("device kernels need block_size 1, 16 or 32 (got %d)", d->block_size);
        return false;
    }
    if (attention && d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256) {
        set_error("attention kernels support head_dim 64, 128 and 256 (got %d)", d->head_dim);
        return false;
    }
    return true;
}

}  // namespace pkv

using namespace pkv;

using Digest = std::array<uint8_t, 32>;

struct DigestHash {
    size_t operator()(const Digest& d) const {
        size_t h;
        std::memcpy(&h, d.data(), sizeof(h));   // SHA-256 output bits are uniform
        return h;
    }
};

// SHA-256(parent || tokens as little-endian int32 || extra as little-endian int64),
// the message assembled in one buffer.
static void chain_hash(const Digest& parent, const int32_t* tokens, int32_t n, int64_t extra,
                       Digest& out) {
    thread_local std::vector<uint8_t> msg;
    msg.resize(32 + 4 * (size_t)n + 8);
    std::memcpy(msg.data(), parent.data(), 32);
    uint8_t* q = msg.data() + 32;
    for (int32_t i = 0; i < n; ++i, q += 4) {
        const uint32_t t = (uint32_t)tokens[i];
        q[0] = (uint8_t)t;
        q[1] = (uint8_t)(t >> 8);
        q[2] = (uint8_t)(t >> 16);
        q[3] = (uint8_t)(t >> 24);
    }
    for (int i = 0; i < 8; ++i) q[i] = (uint8_t)((uint64_t)extra >> (8 * i));
    Sha256 h;
    h.update(msg.data(), msg.size());
    h.final(out.data());
}

// The free-block queue: a doubly linked list threaded through per-block links, so a
// cached block that a new prompt matches can leave from the middle in O(1).
struct FreeQueue {
    std::vector<int32_t> prev, next;
    std::vector<char> queued;
    int32_t head = -1, tail = -1;
    int64_t count = 0;

    void init(const std::vector<int32_t>& order, int32_t nb) {
        prev.assign(nb, -1);
        next.assign(nb, -1);
        queued.assign(nb, 0);
        head = tail = -1;
        count = 0;
        for (int32_t b : order) push_back(b);
    }
    int64_t size() const { return count; }
    int32_t front() const { return head; }
    void push_back(int32_t b) {
        prev[b] = tail;
        next[b] = -1;
        if (tail >= 0) next[tail] = b;
        else head = b;
        tail = b;
        queued[b] = 1;
        ++count;
    }
    void remove(int32_t b) {
        if (prev[b] >= 0) next[prev[b]] = next[b];
        else head = next[b];
        if (next[b] >= 0) prev[next[b]] = prev[b];
        else tail = prev[b];
        prev[b] = next[b] = -1;
        queued[b] = 0;
        --count;
    }
    int32_t pop_front() {
        const int32_t b = head;
        remove(b);
        return b;
    }
};

struct Sequence {
    bool alive = false;
    int32_t length = 0;
    std::vector<int32_t> table;
    // prefix caching: token ids of the partly filled last block, the hash of the last
    // full block, the extra key; `tracked` false once tokens went in without ids
    bool tracked = false;
    std::vector<int32_t> partial;
    Digest last{};
    int64_t extra = 0;
};

struct paged_kv_pool {
    paged_kv_pool_desc desc{};
    void* k = nullptr;
    void* v = nullptr;
    bool owns_buffers = false;
    FreeQueue free_queue;
    std::vector<int32_t> refcount;
    std::vector<Sequence> seqs;
    // prefix caching
    bool prefix = false;
    std::vector<char> has_hash;
    std::vector<Digest> block_digest;
    std::unordered_map<Digest, int32_t, DigestHash> cached;
    int64_t hit_blocks = 0, evictions = 0;
};

// Take the block at the queue head; cached content there leaves the map first.
static int32_t take_free(paged_kv_pool* p) {
    const int32_t b = p->free_queue.pop_front();
    if (p->prefix && p->has_hash[b]) {
        p->cached.erase(p->block_digest[b]);
        p->has_hash[b] = 0;
        ++p->evictions;
    }
    return b;
}

static Sequence* find_seq(paged_kv_pool* p, int32_t id) {
    if (!p || id < 0 || (size_t)id >= p->seqs.size() || !p->seqs[id].alive) return nullptr;
    return &p->seqs[id];
}

static const Sequence* find_seq(const paged_kv_pool* p, int32_t id) {
    return find_seq(const_cast<paged_kv_pool*>(p), id);
}

extern "C" {

const char* paged_kv_status_string(paged_kv_status s) {
    switch (s) {
        case PAGED_KV_OK: return "ok";
        case PAGED_KV_ERR_INVALID_ARG: return "invalid argument";
        case PAGED_KV_ERR_OUT_OF_BLOCKS: return "out of blocks";
        case PAGED_KV_ERR_UNSUPPORTED: return "unsupported";
        case PAGED_KV_ERR_HIP: return "HIP runtime error";
        case PAGED_KV_ERR_NO_SUCH_SEQ: return "no such sequence";
        case PAGED_KV_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    }
    return "unknown status";
}

const char* paged_kv_last_error(void) { return g_last_error.c_str(); }

uint64_t paged_kv_bytes_per_token(int32_t layers, int32_t kv_heads, int32_t head_dim,
                                  int32_t dtype_bytes) {
    if (layers < 0 || kv_heads < 0 || head_dim < 0 || dtype_bytes < 0) return 0;
    return 2ull * (uint64_t)layers * (uint64_t)kv_heads * (uint64_t)head_dim *
           (uint64_t)dtype_bytes;
}

size_t paged_kv_pool_bytes(const paged_kv_pool_desc* d) {
    if (!valid_desc(d)) return 0;
    return (size_t)d->num_blocks * d->num_kv_heads * d->block_size * d->head_dim *
           elem_bytes(d->dtype);
}

paged_kv_status paged_kv_pool_create(const paged_kv_pool_desc* desc, const int32_t* free_order,
                                     void* k_pool, void* v_pool, paged_kv_pool** out) {
    clear_error();
    if (!out) { set_error("null output pointer"); return PAGED_KV_ERR_INVALID_ARG; }
    *out = nullptr;
    if (!valid_desc(desc)) return PAGED_KV_ERR_INVALID_ARG;
    const bool host_only = desc->flags & PAGED_KV_POOL_HOST_ONLY;
    if (!host_only && ((k_pool == nullptr) != (v_pool == nullptr))) {
        set_error("give both k_pool and v_pool, or neither");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    const int32_t nb = desc->num_blocks;
    std::vector<int32_t> order(nb);
    if (free_order) {
        std::vector<char> seen(nb, 0);
        for (int32_t i = 0; i < nb; ++i) {
            int32_t b = free_order[i];
            if (b < 0 || b >= nb || seen[b]) {
                set_error("free_order is not a permutation of 0..%d (entry %d = %d)", nb - 1, i, b);
                return PAGED_KV_ERR_INVALID_ARG;
            }
            seen[b] = 1;
            order[i] = b;
        }
    } else {
        for (int32_t i = 0; i < nb; ++i) order[i] = i;
    }
    auto* p = new paged_kv_pool();
    p->desc = *desc;
    p->free_queue.init(order, nb);
    p->refcount.assign(nb, 0);
    p->prefix = (desc->flags & PAGED_KV_POOL_PREFIX_CACHE) != 0;
    if (p->prefix) {
        p->has_hash.assign(nb, 0);
        p->block_digest.assign(nb, Digest{});
    }
    if (!host_only) {
        if (k_pool) {
            p->k = k_pool;
            p->v = v_pool;
        } else {
            size_t bytes = paged_kv_pool_bytes(desc);
            hipError_t e1 = hipMalloc(&p->k, bytes);
            hipError_t e2 = e1 == hipSuccess ? hipMalloc(&p->v, bytes) : e1;
            if (e1 == hipSuccess && e2 == hipSuccess) {
                e1 = hipMemset(p->k, 0xFF, bytes);
                e2 = e1 == hipSuccess ? hipMemset(p->v, 0xFF, bytes) : e1;
            }
            if (e1 != hipSuccess || e2 != hipSuccess) {
                set_error("pool allocation of 2 x %zu bytes failed: %s", bytes,
                          hipGetErrorString(e1 != hipSuccess ? e1 : e2));
                if (p->k) (void)hipFree(p->k);
                if (p->v) (void)hipFree(p->v);
                delete p;
                return PAGED_KV_ERR_HIP;
            }
            p->owns_buffers = true;
        }
    }
    *out = p;
    return PAGED_KV_OK;
}

void paged_kv_pool_destroy(paged_kv_pool* p) {
    if (!p) return;
    if (p->owns_buffers) {
        (void)hipFree(p->k);
        (void)hipFree(p->v);
    }
    delete p;
}

paged_kv_status paged_kv_pool_buffers(const paged_kv_pool* p, void** k, void** v) {
    clear_error();
    if (!p || !k || !v) { set_error("null argument"); return PAGED_KV_ERR_INVALID_ARG; }
    *k = p->k;
    *v = p->v;
    return PAGED_KV_OK;
}

paged_kv_status paged_kv_pool_get_desc(const paged_kv_pool* p, paged_kv_pool_desc* d) {
    clear_error();
    if (!p || !d) { set_error("null argument"); return PAGED_KV_ERR_INVALID_ARG; }
    *d = p->desc;
    return PAGED_KV_OK;
}

paged_kv_status paged_kv_seq_create(paged_kv_pool* p, int32_t* seq_id) {
    clear_error();
    if (!p || !seq_id) { set_error("null argument"); return PAGED_KV_ERR_INVALID_ARG; }
    if (p->seqs.size() >= (size_t)INT32_MAX) { set_error("sequence ids exhausted"); return PAGED_KV_ERR_INVALID_ARG; }
    p->seqs.emplace_back();
    p->seqs.back().alive = true;
    *seq_id = (int32_t)p->seqs.size() - 1;
    return PAGED_KV_OK;
}

paged_kv_status paged_kv_seq_fork(paged_kv_pool* p, int32_t parent, int32_t* child) {
    clear_error();
    if (!p || !child) { set_error("null argument"); return PAGED_KV_ERR_INVALID_ARG; }
    const Sequence* par = find_seq(p, parent);
    if (!par) { set_error("no live sequence %d", parent); return PAGED_KV_ERR_NO_SUCH_SEQ; }
    Sequence s = *par;
    for (int32_t b : s.table) p->refcount[b] += 1;
    p->seqs.push_back(std::move(s));     // may reallocate: `par` is not used after this
    *child = (int32_t)p->seqs.size() - 1;
    return PAGED_KV_OK;
}

// Blocks an append of n tokens takes from the queue, and whether it copies the tail.
static int64_t blocks_needed(const paged_kv_pool* p, const Sequence& s, int32_t n, bool* cow) {
    const int64_t bs = p->desc.block_size, len = s.length;
    int64_t fresh = (len + n + bs - 1) / bs - (len + bs - 1) / bs;   // offsets 0 in [len, len+n)
    *cow = n > 0 && (len % bs) != 0 && p->refcount[s.table.back()] > 1;
    return fresh + (*cow ? 1 : 0);
}

static paged_kv_status append_one(paged_kv_pool* p, int32_t seq, int32_t n, int32_t* slots_out,
                                  int32_t* copies_out, int32_t max_copies, int32_t* n_copies,
                                  const int32_t* tokens = nullptr) {
    Sequence* s = find_seq(p, seq);
    if (!s) { set_error("no live sequence %d", seq); return PAGED_KV_ERR_NO_SUCH_SEQ; }
    if (n < 0) { set_error("n_tokens %d < 0", n); return PAGED_KV_ERR_INVALID_ARG; }
    if ((int64_t)s->length + n > INT32_MAX) { set_error("sequence length overflow"); return PAGED_KV_ERR_INVALID_ARG; }
    bool cow = false;
    int64_t need = blocks_needed(p, *s, n, &cow);
    if (need > (int64_t)p->free_queue.size()) {
        set_error("sequence %d needs %lld blocks, %lld free", seq, (long long)need,
                  (long long)p->free_queue.size());
        return PAGED_KV_ERR_OUT_OF_BLOCKS;
    }
    if (cow && max_copies < 1) {
        set_error("append of sequence %d copies a shared block; copies buffer holds %d pairs",
                  seq, max_copies);
        return PAGED_KV_ERR_BUFFER_TOO_SMALL;
    }
    *n_copies = 0;
    const int32_t bs = p->desc.block_size;
    if (!tokens) s->tracked = false;
    if (cow) {
        int32_t src = s->table.back();
        int32_t dst = take_free(p);
        p->refcount[src] -= 1;
        p->refcount[dst] = 1;
        s->table.back() = dst;
        copies_out[0] = src;
        copies_out[1] = dst;
        *n_copies = 1;
    }
    for (int32_t i = 0; i < n; ++i) {
        int32_t pos = s->length;
        if (pos % bs == 0) {
            int32_t b = take_free(p);
            p->refcount[b] = 1;
            s->table.push_back(b);
        }
        slots_out[i] = s->table[pos / bs] * bs + pos % bs;
        s->length = pos + 1;
        if (s->tracked) {
            s->partial.push_back(tokens[i]);
            if ((int32_t)s->partial.size() == bs) {   // the block just became full
                chain_hash(s->last, s->partial.data(), bs, s->extra, s->last);
                s->partial.clear();
                const int32_t b = s->table[pos / bs];
                if (!p->has_hash[b] && p->cached.find(s->last) == p->cached.end()) {
                    p->cached.emplace(s->last, b);
                    p->block_digest[b] = s->last;
                    p->has_hash[b] = 1;
                }
            }
        }
    }
    return PAGED_KV_OK;
}

paged_kv_status paged_kv_seq_append(paged_kv_pool* p, int32_t seq, int32_t n_tokens,
                                    int32_t* slots_out, int32_t* copies_out, int32_t max_copies,
                                    int32_t* n_copies) {
    clear_error();
    if (!p || !n_copies || (n_tokens > 0 && !slots_out) || (max_copies > 0 && !copies_out)) {
        set_error("null argument");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    *n_copies = 0;
    return append_one(p, seq, n_tokens, slots_out, copies_out, max_copies, n_copies);
}

paged_kv_status paged_kv_append_batch(paged_kv_pool* p, const int32_t* seqs, const int32_t* counts,
                                      int32_t n_seqs, int32_t* slots_out, int32_t* copies_out,
                                      int32_t max_copies, int32_t* n_copies, int32_t* n_done) {
    clear_error();
    if (!p || !n_copies || !n_done || n_seqs < 0 || (n_seqs > 0 && (!seqs || !counts)) ||
        (max_copies > 0 && !copies_out)) {
        set_error("null or invalid argument");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    *n_copies = 0;
    *n_done = 0;
    int64_t slot_pos = 0;
    for (int32_t i = 0; i < n_seqs; ++i) {
        if (counts[i] > 0 && !slots_out) { set_error("null slots_out"); return PAGED_KV_ERR_INVALID_ARG; }
        int32_t nc = 0;
        paged_kv_status st = append_one(p, seqs[i], counts[i], slots_out ? slots_out + slot_pos : nullptr,
                                        copies_out ? copies_out + 2 * (*n_copies) : nullptr,
                                        max_copies - *n_copies, &nc);
        if (st != PAGED_KV_OK) return st;
        slot_pos += counts[i];
        *n_copies += nc;
        *n_done = i + 1;
    }
    return PAGED_KV_OK;
}

paged_kv_status paged_kv_block_hash(const uint8_t* parent, const int32_t* tokens, int32_t n,
                                    int64_t extra_key, uint8_t* out) {
    clear_error();
    if (!out || n < 0 || (n > 0 && !tokens)) { set_error("null or invalid argument"); return PAGED_KV_ERR_INVALID_ARG; }
    Digest par{}, d;
    if (parent) std::memcpy(par.data(), parent, 32);
    chain_hash(par, tokens, n, extra_key, d);
    std::memcpy(out, d.data(), 32);
    return PAGED_KV_OK;
}

paged_kv_status paged_kv_seq_create_prefix(paged_kv_pool* p, const int32_t* prompt, int32_t n,
                                           int64_t extra_key, int32_t* seq_id, int32_t* n_cached) {
    clear_error();
    if (!p || !seq_id || !n_cached || n < 0 || (n > 0 && !prompt)) {
        set_error("null or invalid argument");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    if (!p->prefix) { set_error("pool was created without PAGED_KV_POOL_PREFIX_CACHE"); return PAGED_KV_ERR_UNSUPPORTED; }
    if (p->seqs.size() >= (size_t)INT32_MAX) { set_error("sequence ids exhausted"); return PAGED_KV_ERR_INVALID_ARG; }
    Sequence s;
    s.alive = true;
    s.tracked = true;
    s.extra = extra_key;
    const int32_t bs = p->desc.block_size;
    const int32_t full = n > 0 ? (n - 1) / bs : 0;      // the last prompt token is recomputed
    for (int32_t i = 0; i < full; ++i) {
        Digest h;
        chain_hash(s.last, prompt + (int64_t)i * bs, bs, extra_key, h);
        auto it = p->cached.find(h);
        if (it == p->cached.end()) break;
        const int32_t b = it->second;
        if (p->refcount[b] == 0) p->free_queue.remove(b);
        p->refcount[b] += 1;
        s.table.push_back(b);
        s.length += bs;
        s.last = h;
        ++p->hit_blocks;
    }
    p->seqs.push_back(std::move(s));
    *seq_id = (int32_t)p->seqs.size() - 1;
    *n_cached = p->seqs.back().length;
    return PAGED_KV_OK;
}

paged_kv_status paged_kv_seq_append_tokens(paged_kv_pool* p, int32_t seq, const int32_t* tokens,
                                           int32_t n_tokens, int32_t* slots_out,
                                           int32_t* copies_out, int32_t max_copies,
                                           int32_t* n_copies) {
    clear_error();
    if (!p || !n_copies || (n_tokens > 0 && (!slots_out || !tokens)) || (max_copies > 0 && !copies_out)) {
        set_error("null argument");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    *n_copies = 0;
    static const int32_t none = 0;
    return append_one(p, seq, n_tokens, slots_out, copies_out, max_copies, n_copies,
                      n_tokens > 0 ? tokens : &none);
}

paged_kv_status paged_kv_prefix_stats(const paged_kv_pool* p, int64_t* cached_blocks,
                                      int64_t* hit_blocks, int64_t* evictions) {
    clear_error();
    if (!p || !cached_blocks || !hit_blocks || !evictions) { set_error("null argument"); return PAGED_KV_ERR_INVALID_ARG; }
    *cached_blocks = (int64_t)p->cached.size();
    *hit_blocks = p->hit_blocks;
    *evictions = p->evictions;
    return PAGED_KV_OK;
}

paged_kv_status paged_kv_seq_free(paged_kv_pool* p, int32_t seq) {
    clear_error();
    Sequence* s = find_seq(p, seq);
    if (!s) { set_error("no live sequence %d", seq); return PAGED_KV_ERR_NO_SUCH_SEQ; }
    for (int32_t b : s->table) {
        if (--p->refcount[b] == 0) p->free_queue.push_back(b);
    }
    s->alive = false;
    s->length = 0;
    std::vector<int32_t>().swap(s->table);
    return PAGED_KV_OK;
}

paged_kv_status paged_kv_block_tables(const paged_kv_pool* p, const int32_t* ids, int32_t n,
                                      int32_t max_blocks, int32_t* tables_out,
                                      int32_t* lens_out) {
    clear_error();
    if (!p || n < 0 || max_blocks < 0 || (n > 0 && (!ids || !lens_out || (max_blocks > 0 && !tables_out)))) {
        set_error("null or invalid argument");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    for (int32_t i = 0; i < n; ++i) {
        const Sequence* s = find_seq(p, ids[i]);
        if (!s) { set_error("no live sequence %d", ids[i]); return PAGED_KV_ERR_NO_SUCH_SEQ; }
        if ((int64_t)s->table.size() > max_blocks) {
            set_error("sequence %d has %zu blocks, table width %d", ids[i], s->table.size(), max_blocks);
            return PAGED_KV_ERR_INVALID_ARG;
        }
    }
    for (int32_t i = 0; i < n; ++i) {
        const Sequence* s = find_seq(p, ids[i]);
        int32_t* row = tables_out + (int64_t)i * max_blocks;
        int32_t j = 0;
        for (; j < (int32_t)s->table.size(); ++j) row[j] = s->table[j];
        for (; j < max_blocks; ++j) row[j] = -1;
        lens_out[i] = s->length;
    }
    return PAGED_KV_OK;
}

paged_kv_status paged_kv_seq_info(const paged_kv_pool* p, int32_t seq, int32_t* len,
                                  int32_t* nblocks) {
    clear_error();
    if (!len || !nblocks) { set_error("null argument"); return PAGED_KV_ERR_INVALID_ARG; }
    const Sequence* s = find_seq(p, seq);
    if (!s) { set_error("no live sequence %d", seq); return PAGED_KV_ERR_NO_SUCH_SEQ; }
    *len = s->length;
    *nblocks = (int32_t)s->table.size();
    return PAGED_KV_OK;
}

paged_kv_status paged_kv_block_refcount(const paged_kv_pool* p, int32_t block, int32_t* rc) {
    clear_error();
    if (!p || !rc || block < 0 || block >= p->desc.num_blocks) {
        set_error("null argument or block %d out of range", block);
        return PAGED_KV_ERR_INVALID_ARG;
    }
    *rc = p->refcount[block];
    return PAGED_KV_OK;
}

paged_kv_status paged_kv_stats(const paged_kv_pool* p, int64_t* num_free, int64_t* num_used,
                               int64_t* waste) {
    clear_error();
    if (!p || !num_free || !num_used || !waste) { set_error("null argument"); return PAGED_KV_ERR_INVALID_ARG; }
    *num_free = (int64_t)p->free_queue.size();
    *num_used = p->desc.num_blocks - *num_free;
    int64_t w = 0;
    for (const Sequence& s : p->seqs)
        if (s.alive) w += (int64_t)p->desc.block_size * (int64_t)s.table.size() - s.length;
    *waste = w;
    return PAGED_KV_OK;
}

paged_kv_status paged_kv_shared_prefix_groups(const paged_kv_pool* p, const int32_t* seq_ids,
                                              int32_t n, int32_t max_group,
                                              int32_t min_shared_tokens, int32_t* group_start_out,
                                              int32_t* shared_tokens_out, int32_t* num_groups_out,
                                              int32_t* max_shared_out) {
    clear_error();
    if (!p || n < 0 || max_group < 1 || (n > 0 && (!seq_ids || !group_start_out ||
                                                    !shared_tokens_out)) ||
        !num_groups_out || !max_shared_out) {
        set_error("null pointer, n < 0 or max_group < 1");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    std::vector<const Sequence*> seqs(n);
    for (int32_t i = 0; i < n; ++i) {
        seqs[i] = find_seq(p, seq_ids[i]);
        if (!seqs[i]) { set_error("no sequence %d", seq_ids[i]); return PAGED_KV_ERR_NO_SUCH_SEQ; }
    }
    const int64_t bs = p->desc.block_size;
    const int64_t need = std::max<int64_t>(1, min_shared_tokens);
    int32_t g = 0, max_shared = 0;
    for (int32_t i = 0; i < n;) {
        // grow the group while the tokens shared by all of its members stay >= need
        const std::vector<int32_t>& first = seqs[i]->table;
        int64_t common = (int64_t)first.size(), min_len = seqs[i]->length;
        int32_t j = i + 1;
        for (; j < n && j - i < max_group; ++j) {
            const std::vector<int32_t>& t = seqs[j]->table;
            int64_t c = 0;
            const int64_t lim = std::min<int64_t>(common, (int64_t)t.size());
            while (c < lim && t[c] == first[c]) ++c;
            const int64_t len = std::min<int64_t>(min_len, seqs[j]->length);
            if (std::min(c * bs, len) < need) break;
            common = c;
            min_len = len;
        }
        const int32_t shared = j - i > 1 ? (int32_t)std::min(common * bs, min_len) : 0;
        group_start_out[g] = i;
        shared_tokens_out[g] = shared;
        max_shared = std::max(max_shared, shared);
        ++g;
        i = j;
    }
    if (n > 0) group_start_out[g] = n;
    else if (group_start_out) group_start_out[0] = 0;
    *num_groups_out = g;
    *max_shared_out = max_shared;
    return PAGED_KV_OK;
}

}  // extern "C"
