// Paged decode attention for batches whose sequences share a prompt prefix (gfx950).
//
// Parallel sampling (deepsonar "PagedAttention de vLLM …" §2.3: the samples of one
// prompt share its blocks through reference counts and copy only the block they write;
// deeplearn.tn "PagedAttention : comment optimiser la mémoire GPU …", concrete benefits
// section: flexible sharing of the KV cache) leaves the prompt's K/V stored once while
// every sample attends over it.  Attending sample by sample reads the shared blocks once
// per sample.  Here the shared part is read once per group: its tiles are multiplied
// against the queries of all the group's samples together (the group's samples times the
// query heads of a KV head form the N side of the MFMA tiles, up to 64 slots), and each
// sample's own tail is attended separately; a merge launch then combines, per sample and
// query head, the prefix partitions with the tail partitions by log-sum-exp.  What is
// computed is unchanged: softmax attention over the whole context of each sequence.
//
// Work items, one per workgroup (its four waves take the item's tiles in turn and merge
// their states in LDS):
//   prefix item (group, KV head, partition p of the shared tokens): tokens
//     [p PT, min((p + 1) PT, shared)), read through the table of the group's first
//     member; the other members' table entries for those tokens are checked equal (a
//     mismatch makes the group's results NaN);
//   tail item (sequence, KV head, partition p of its own tokens): tokens
//     [max(shared, j PT), min((j + 1) PT, ctx)) with j = floor(shared / PT) + p; the
//     sequence's first tail item also writes what the merge needs to know of it (its
//     number of partition states, or 0 where the group description does not hold).
// Each item writes the raw (max, sum, weighted values) state of every query head it
// serves into the workspace row (sequence, query head, partition index), where prefix
// partitions come first and tail partitions follow; the merge folds them in order.
// Only the logical token order decides the summation order, so placement in the pool
// does not change the results.

#include <algorithm>

#include "attention_common.h"

namespace {

using namespace pkv_dev;

struct SharedArgs {
    void* out;
    const void* q;
    const void* k_pool;
    const void* v_pool;
    const int32_t* block_tables;
    const int32_t* context_lens;
    const int32_t* group_start;     // [num_groups + 1]
    const int32_t* shared_tokens;   // [num_groups]
    i32x4* seq_desc;                // [num_seqs]: what the merge needs to know of each sequence
    float* ws_m;
    float* ws_l;
    float* ws_acc;
    int32_t num_seqs;
    int32_t num_groups;
    int32_t max_group;              // host bound on members per group
    int32_t members_per_item;       // members one prefix item serves (16 NB / G)
    int32_t chunks;                 // prefix items per (group, KV head, partition)
    int32_t max_blocks_per_seq;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;                  // query heads per KV head (G)
    int32_t num_blocks;
    int32_t max_context_len;
    int32_t partition_tokens;       // PT
    int32_t max_shared;             // host bound on every shared_tokens[g]
    int32_t block_size;
    int32_t prefix_parts;           // partitions of the longest shared prefix (host bound)
    int32_t tail_parts;             // partitions of the longest tail (host bound)
    int32_t max_parts;              // workspace rows per (sequence, query head)
    int64_t prefix_items;           // num_groups * Hkv * prefix_parts
    int64_t items;                  // prefix_items + num_seqs * Hkv * tail_parts
    float scale_log2;
};

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Group of sequence s: the number of g in [1, num_groups) with group_start[g] <= s, which
// for a non-decreasing group_start is the last group starting at or before s.  The lanes
// of a wave compare 64 group starts per memory round trip (instead of a chain of
// dependent scalar loads).  Every kernel that needs the group of a sequence uses this.
__device__ __forceinline__ int group_of(const SharedArgs& a, int s) {
    const int lane = threadIdx.x & 63;
    int cnt = 0;
    for (int g0 = 1; g0 < a.num_groups; g0 += 64) {
        const int g = g0 + lane;
        const bool le = g < a.num_groups && a.group_start[g] <= s;
        cnt += __popcll(__ballot(le));
    }
    return cnt;
}

// One workgroup per item; wave w takes the item's tiles w, w + 4, w + 8, ...  NB N-blocks
// of 16 query slots (slot n = member * G + head of the KV head's group for a prefix item;
// n = head for a tail item, which uses N-block 0 only).
template <int D, int DT, int BS, int NB>
__global__ __launch_bounds__(kWaves * 64)
__attribute__((amdgpu_waves_per_eu(NB == 1 ? mfma_waves_per_simd<D, false>() : NB * D <= 256 ? 2 : 1)))
void attn_mfma_shared(SharedArgs a) {
    constexpr int KI = D / 32;
    constexpr int MT = D / 16;
    constexpr int TILE = BS * D;
    constexpr int TPB = BS / kTile;
    using kvec = typename std::conditional<DT == DT_BF16, bf16x8, f16x8>::type;
    static_assert(BS >= kTile, "16- and 32-token blocks only");

    const int lane = threadIdx.x & 63;
    const int w = uni(threadIdx.x >> 6);
    const int64_t item = blockIdx.x;
    // (every return before the merge below depends on the item alone: the whole
    // workgroup takes it)
    if (item >= a.items) return;
    const int gq = lane & 15, quad = lane >> 4;
    const int G = a.group;

    // ---- decode the item ----
    bool prefix;
    int s0, members, h, p, start, end, part_index;
    bool bad = false;
    int lead = 0;   // batch row whose table the item reads through
    if (item < a.prefix_items) {
        // (group, KV head, partition, chunk of members): a group larger than one item's
        // N side is served by several items, each reading the shared tiles through the
        // group's first table (so the merge's check against that table covers them all)
        prefix = true;
        const int per_group = a.num_kv_heads * a.prefix_parts * a.chunks;
        const int g = (int)(item / per_group);
        int r = (int)(item - (int64_t)g * per_group);
        const int c = r % a.chunks;
        r /= a.chunks;
        h = r / a.prefix_parts;
        p = r - h * a.prefix_parts;
        lead = sload(a.group_start, g);
        const int gsize = sload(a.group_start, g + 1) - lead;
        const int shared = sload(a.shared_tokens, g);
        if (shared < 0 || shared > a.max_shared) return;   // the merge gives the group NaN
        start = p * a.partition_tokens;
        end = min(start + a.partition_tokens, shared);
        // a malformed group range is never read through (the merge gives its rows NaN)
        if (gsize < 1 || start >= end || lead < 0 || lead + gsize > a.num_seqs) return;
        if (gsize > a.max_group) bad = true;
        s0 = lead + c * a.members_per_item;
        members = min(a.members_per_item, min(gsize, a.max_group) - c * a.members_per_item);
        if (members < 1) return;
        part_index = p;
    } else {
        // Tail items partition-major: every sequence's first tail partition comes first,
        // and the (mostly empty) later ones follow together at the end of the grid.  Tail
        // partitions sit at absolute multiples of PT ([max(shared, j PT), (j + 1) PT) for
        // j >= shared / PT), so a tile never straddles two of them.
        prefix = false;
        const int64_t t = item - a.prefix_items;
        const int64_t per_part = (int64_t)a.num_seqs * a.num_kv_heads;
        p = (int)(t / per_part);
        const int r = (int)(t - (int64_t)p * per_part);
        s0 = r / a.num_kv_heads;
        h = r - s0 * a.num_kv_heads;
        members = 1;
        const int g = group_of(a, s0);
        const int shared = sload(a.shared_tokens, g);
        const int ctx = sload(a.context_lens, s0);
        const int PT = a.partition_tokens;
        if (h == 0 && p == 0) {
            // The sequence's descriptor for the merge: its number of partition states,
            // its group's first row and the blocks the shared tokens span (whose ids its
            // table must repeat), or 0 states if the group description does not hold for
            // it (the merge then writes NaN).
            const int gs = sload(a.group_start, g), ge = sload(a.group_start, g + 1);
            const bool valid = ctx >= 1 && ctx <= a.max_context_len && shared >= 0 &&
                               shared <= ctx && shared <= a.max_shared && gs >= 0 &&
                               ge <= a.num_seqs && s0 >= gs && s0 < ge && s0 - gs < a.max_group;
            if (threadIdx.x == 0) {
                const int np = (shared + PT - 1) / PT +
                               (ctx > shared ? (ctx + PT - 1) / PT - shared / PT : 0);
                a.seq_desc[s0] = valid ? (i32x4){np, gs, (shared + a.block_size - 1) / a.block_size, 0}
                                       : (i32x4){0, 0, 0, 0};
            }
        }
        // invalid lengths: nothing to read here (the merge gives the rows NaN)
        if (ctx < 1 || ctx > a.max_context_len || shared < 0 || shared > ctx ||
            shared > a.max_shared) return;
        const int j0 = shared / PT;
        const int jb = j0 + p;   // absolute partition (token / PT)
        start = max(shared, jb * PT);
        end = min((jb + 1) * PT, ctx);
        if (start >= end) return;
        part_index = (shared + PT - 1) / PT + (jb - j0);
        lead = s0;
    }
    const int slots = members * G;                 // query slots of this item
    const int nb_used = (slots + 15) / 16;
    const int32_t* trow = a.block_tables + (int64_t)lead * a.max_blocks_per_seq;

    // A prefix item reads the group's shared blocks through the first member's table; that
    // every member's length covers them and its table lists the same blocks is checked by
    // the merge, which gives the member NaN otherwise (checking here would hold up the
    // first loads by a memory round trip per member).
    (void)prefix;

    // ---- queries: N-block nb, lane slot n = 16 nb + gq -> (member n / G, head n % G) ----
    kvec qop[NB][KI];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int n = min(16 * nb + gq, slots - 1);    // padded slots repeat the last one
        const int m = n / G, j = n - m * G;
        const uint16_t* qh = static_cast<const uint16_t*>(a.q) +
                             ((int64_t)(s0 + m) * a.num_q_heads + h * G + j) * D + 8 * quad;
#pragma unroll
        for (int kk = 0; kk < KI; ++kk)
            qop[nb][kk] = __builtin_bit_cast(kvec, *reinterpret_cast<const i32x4*>(qh + 32 * kk));
    }

    const uint16_t* kpool = static_cast<const uint16_t*>(a.k_pool) + (int64_t)h * TILE;
    const uint16_t* vpool = static_cast<const uint16_t*>(a.v_pool) + (int64_t)h * TILE;
    const int64_t blk_stride = (int64_t)a.num_kv_heads * TILE;
    const int voff = gq * 4 + quad;

    f32x4 acc[NB][MT];
    float m_run[NB], lsum[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nb][mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
        m_run[nb] = kNegInf;
        lsum[nb] = 0.f;
    }

    const int t_begin = start / kTile, t_end = (end + kTile - 1) / kTile;
    const int n = t_end - t_begin;

    auto load = [&](int it, i32x4 (&kr)[KI], i32x2 (&vr)[MT]) __attribute__((always_inline)) {
        int32_t bid = sload(trow, it / TPB);
        if ((uint32_t)bid >= (uint32_t)a.num_blocks) {
            bad = true;
            bid = 0;
        }
        const int64_t base = (int64_t)bid * blk_stride + (it % TPB) * (kTile * D);
        const i32x4* kt = reinterpret_cast<const i32x4*>(kpool + base) + lane;
        const i32x2* vt = reinterpret_cast<const i32x2*>(vpool + base) + voff;
#pragma unroll
        for (int kk = 0; kk < KI; ++kk) kr[kk] = __builtin_nontemporal_load(kt + kk * 64);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) vr[mt] = __builtin_nontemporal_load(vt + mt * 64);
    };

    auto compute = [&](int it, const i32x4 (&kr)[KI], i32x2 (&vr)[MT]) __attribute__((always_inline)) {
        const int valid = min(kTile, end - it * kTile);   // tokens of the tile in range
        const int first = max(0, start - it * kTile);     // (start is a tile boundary unless
                                                          // a tail begins mid-tile)
        const int tok0 = 4 * quad;
        if (valid < kTile || first > 0) {
            // slots outside [start, end) may hold anything (NaN included): clear them
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                uint32_t lo = (uint32_t)vr[mt][0], hi = (uint32_t)vr[mt][1];
                if (tok0 + 0 >= valid || tok0 + 0 < first) lo &= 0xFFFF0000u;
                if (tok0 + 1 >= valid || tok0 + 1 < first) lo &= 0x0000FFFFu;
                if (tok0 + 2 >= valid || tok0 + 2 < first) hi &= 0xFFFF0000u;
                if (tok0 + 3 >= valid || tok0 + 3 < first) hi &= 0x0000FFFFu;
                vr[mt][0] = (int)lo;
                vr[mt][1] = (int)hi;
            }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            if (nb >= nb_used) break;
            f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KI; ++kk) {
                if constexpr (DT == DT_BF16)
                    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[kk]),
                                                                 qop[nb][kk], sc, 0, 0, 0);
                else
                    sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, kr[kk]),
                                                                qop[nb][kk], sc, 0, 0, 0);
            }
            float x[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                x[j] = (tok0 + j < valid && tok0 + j >= first) ? sc[j] * a.scale_log2 : kNegInf;
            // lazy rescaling (the reference max moves only past a slack of 2^8)
            const float xm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
            if (__ballot(xm > m_run[nb] + kRescaleSlack)) {
                const float mnew = fmaxf(m_run[nb], max_across_quads(xm));
                const float alpha = exp2_fast(m_run[nb] - mnew);
                lsum[nb] *= alpha;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[nb][mt] *= alpha;
                m_run[nb] = mnew;
            }
            // weights as a 16-bit head and a 16-bit remainder (as in the other decode
            // kernels: one 16-bit rounding of p alone is too coarse for short contexts)
            s16x4 phi, plo;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float pf = exp2_fast(x[j] - m_run[nb]);
                const uint16_t hi = f32_to_bits16<DT>(pf);
                const uint16_t lo = f32_to_bits16<DT>(pf - bits_to_f32<DT>(hi));
                phi[j] = (short)hi;
                plo[j] = (short)lo;
                lsum[nb] += pf;
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if constexpr (DT == DT_BF16) {
                    const s16x4 va = __builtin_bit_cast(s16x4, vr[mt]);
                    acc[nb][mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, phi, acc[nb][mt], 0, 0, 0);
                    acc[nb][mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, plo, acc[nb][mt], 0, 0, 0);
                } else {
                    const f16x4 va = __builtin_bit_cast(f16x4, vr[mt]);
                    acc[nb][mt] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, __builtin_bit_cast(f16x4, phi),
                                                                       acc[nb][mt], 0, 0, 0);
                    acc[nb][mt] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, __builtin_bit_cast(f16x4, plo),
                                                                       acc[nb][mt], 0, 0, 0);
                }
            }
        }
    };

    // Wave w's tiles: t_begin + w + 4 i.  Two register sets: the next tile's loads are in
    // flight while the current one is computed.
    const int n_w = n > w ? (n - w + kWaves - 1) / kWaves : 0;
    i32x4 kA[KI], kB[KI];
    i32x2 vA[MT], vB[MT];
    const int t0 = t_begin + w;
    if (n_w > 0) load(t0, kA, vA);
    int i = 0;
    for (; i + 2 < n_w; i += 2) {
        load(t0 + kWaves * (i + 1), kB, vB);
        __builtin_amdgcn_sched_barrier(0);
        compute(t0 + kWaves * i, kA, vA);
        load(t0 + kWaves * (i + 2), kA, vA);
        __builtin_amdgcn_sched_barrier(0);
        compute(t0 + kWaves * (i + 1), kB, vB);
    }
    if (i + 1 < n_w) {
        load(t0 + kWaves * (i + 1), kB, vB);
        __builtin_amdgcn_sched_barrier(0);
        compute(t0 + kWaves * i, kA, vA);
        compute(t0 + kWaves * (i + 1), kB, vB);
    } else if (i < n_w) {
        compute(t0 + kWaves * i, kA, vA);
    }

    // ---- merge the four waves' states (fixed order), write the item's state ----
    constexpr int NS = NB * 16;
    __shared__ float sm_m[kWaves][NS];
    __shared__ float sm_l[kWaves][NS];
    __shared__ float sm_acc[NS][D + 4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const float lw = sum_across_quads(lsum[nb]);
        if (lane < 16) {
            sm_m[w][16 * nb + lane] = m_run[nb];
            sm_l[w][16 * nb + lane] = lw;
        }
    }
    const bool any_bad = __syncthreads_or(bad);
    float f[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        float mmax = kNegInf;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) mmax = fmaxf(mmax, sm_m[ww][16 * nb + gq]);
        f[nb] = m_run[nb] == kNegInf ? 0.f : exp2_fast(m_run[nb] - mmax);
    }
    for (int ww = 0; ww < kWaves; ++ww) {
        if (ww == w) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                if (nb >= nb_used) break;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int d = 16 * mt + 4 * quad + r;
                        const float v = acc[nb][mt][r] * f[nb];
                        if (ww == 0) sm_acc[16 * nb + gq][d] = v;
                        else sm_acc[16 * nb + gq][d] += v;
                    }
            }
        }
        __syncthreads();
    }
    for (int x = threadIdx.x; x < slots * D; x += kWaves * 64) {
        const int sl = x / D, d = x - sl * D;
        float mm = kNegInf;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) mm = fmaxf(mm, sm_m[ww][sl]);
        float l = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww)
            if (sm_m[ww][sl] != kNegInf) l += exp2_fast(sm_m[ww][sl] - mm) * sm_l[ww][sl];
        const int m = sl / G, j = sl - m * G;
        const int64_t row = ((int64_t)(s0 + m) * a.num_q_heads + h * G + j) * a.max_parts + part_index;
        a.ws_acc[row * D + d] = any_bad ? NAN : sm_acc[sl][d];
        if (d == 0) {
            a.ws_m[row] = any_bad ? NAN : mm;
            a.ws_l[row] = any_bad ? NAN : l;
        }
    }
}

// ---------------------------------------------------------------------------------
// Merge: per (sequence, query head), the ceil(shared / PT) prefix partitions and the tail
// partitions (ceil(ctx / PT) - floor(shared / PT) of them), in that order, by an online
// log-sum-exp
//   M' = max(M, m_i), L' = L 2^(M - M') + l_i 2^(m_i - M'), acc likewise; out = acc / L.
// One workgroup per (sequence, KV head); each thread merges kMergeOut outputs (head dims of
// the KV head's query heads), all their partitions' loads in flight together.
// ---------------------------------------------------------------------------------
constexpr int kMergeOut = 2;

// KP: partitions folded per memory round trip (2 or 4 when no sequence has more, else 8;
// past a sequence's last partition the slots re-read it).
template <int D, int OUT_DT, int KP>
__global__ __launch_bounds__(1024) void attn_shared_merge(SharedArgs a) {
    const int hk = blockIdx.x, s = blockIdx.y;
    const int G = a.group, n_out = G * D;
    const int64_t obase = ((int64_t)s * a.num_q_heads + hk * G) * D;
    // written by the sequence's first tail item (np = 0: the group description does not
    // hold for it, NaN)
    const int32_t* dsc = reinterpret_cast<const int32_t*>(a.seq_desc + s);
    const int np = sload(dsc, 0), gs = sload(dsc, 1), nblk = s == gs ? 0 : sload(dsc, 2);
    if (np < 1) {
        for (int i = threadIdx.x; i < n_out; i += blockDim.x) store_out<OUT_DT>(a.out, obase + i, NAN);
        return;
    }
    // The shared tokens were read through the group's first table: this sequence's table
    // must list the same blocks for them.  Its entries are loaded together with the first
    // partitions' states, and compared once both are in flight.
    const int32_t* mine = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    const int32_t* first = a.block_tables + (int64_t)gs * a.max_blocks_per_seq;
    bool diff = false;
    for (int i0 = threadIdx.x * kMergeOut; i0 < n_out; i0 += blockDim.x * kMergeOut) {
        float M[kMergeOut], l[kMergeOut], acc[kMergeOut];
        bool bad[kMergeOut];
        int64_t row[kMergeOut];
        int dd[kMergeOut];
#pragma unroll
        for (int u = 0; u < kMergeOut; ++u) {
            const int i = min(i0 + u, n_out - 1);   // (past the end: repeat, not stored)
            row[u] = ((int64_t)s * a.num_q_heads + hk * G + i / D) * a.max_parts;
            dd[u] = i % D;
            M[u] = kNegInf;
            l[u] = 0.f;
            acc[u] = 0.f;
            bad[u] = false;
        }
        for (int p0 = 0; p0 < np; p0 += KP) {
            float mv[kMergeOut][KP], lv[kMergeOut][KP], av[kMergeOut][KP];
#pragma unroll
            for (int u = 0; u < kMergeOut; ++u)
#pragma unroll
                for (int k = 0; k < KP; ++k) {   // slots past the end re-read the last
                    const int64_t r = row[u] + min(p0 + k, np - 1);
                    mv[u][k] = a.ws_m[r];
                    lv[u][k] = a.ws_l[r];
                    av[u][k] = a.ws_acc[r * D + dd[u]];
                }
            if (p0 == 0 && i0 == threadIdx.x * kMergeOut)
                for (int b = threadIdx.x; b < nblk; b += blockDim.x) diff |= mine[b] != first[b];
#pragma unroll
            for (int u = 0; u < kMergeOut; ++u)
#pragma unroll
                for (int k = 0; k < KP; ++k) {
                    if (p0 + k >= np) break;
                    bad[u] |= mv[u][k] != mv[u][k];
                    const float mn = fmaxf(M[u], mv[u][k]);
                    const float sc = exp2_fast(M[u] - mn), w = exp2_fast(mv[u][k] - mn);
                    l[u] = l[u] * sc + w * lv[u][k];
                    acc[u] = acc[u] * sc + w * av[u][k];
                    M[u] = mn;
                }
        }
#pragma unroll
        for (int u = 0; u < kMergeOut; ++u) {
            // the table comparison is only known at the end: store the result (NaN if any
            // partition held one) and overwrite it below if the tables differ
            if (i0 + u < n_out) store_out<OUT_DT>(a.out, obase + i0 + u, bad[u] ? NAN : acc[u] / l[u]);
        }
    }
    // (each thread overwrites its own outputs: program order makes NaN the final value)
    if (__syncthreads_or(diff))
        for (int i0 = threadIdx.x * kMergeOut; i0 < n_out; i0 += blockDim.x * kMergeOut)
#pragma unroll
            for (int u = 0; u < kMergeOut; ++u)
                if (i0 + u < n_out) store_out<OUT_DT>(a.out, obase + i0 + u, NAN);
}

// ---------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct SharedPlan {
    SharedArgs a;
    int nb;          // N-blocks: ceil(max_group * G / 16), 1, 2 or 4
    size_t ws_bytes;
};

int n_blocks_for(int max_group, int group) {
    const int slots = max_group * group;
    return slots <= 16 ? 1 : slots <= 32 ? 2 : slots <= 64 ? 4 : 0;
}

// Workspace: sequence descriptors: int32[num_seqs][4] | m, l: float[rows] |
// acc: float[rows][d], rows = num_seqs * hq * max_parts.  Scratch: every call writes what
// it reads.
size_t desc_region(int64_t num_seqs) { return align256((size_t)num_seqs * 4 * sizeof(int32_t)); }
size_t shared_workspace(int64_t num_seqs, int64_t hq, int64_t d, int64_t max_parts) {
    const size_t rows = (size_t)num_seqs * hq * max_parts;
    return desc_region(num_seqs) + 2 * align256(rows * sizeof(float)) + rows * d * sizeof(float);
}

template <int D, int DT, int BS>
void launch_items(const SharedPlan& pl, dim3 grid, hipStream_t st) {
    switch (pl.nb) {
        case 1: attn_mfma_shared<D, DT, BS, 1><<<grid, dim3(kWaves * 64), 0, st>>>(pl.a); break;
        case 2: attn_mfma_shared<D, DT, BS, 2><<<grid, dim3(kWaves * 64), 0, st>>>(pl.a); break;
        default: attn_mfma_shared<D, DT, BS, 4><<<grid, dim3(kWaves * 64), 0, st>>>(pl.a); break;
    }
}

template <int D, int KP>
void launch_merge(const SharedPlan& pl, int out_dtype, dim3 grid, dim3 block, hipStream_t st) {
    if (out_dtype == PAGED_KV_F32) attn_shared_merge<D, DT_F32, KP><<<grid, block, 0, st>>>(pl.a);
    else if (out_dtype == PAGED_KV_F16) attn_shared_merge<D, DT_F16, KP><<<grid, block, 0, st>>>(pl.a);
    else attn_shared_merge<D, DT_BF16, KP><<<grid, block, 0, st>>>(pl.a);
}

template <int D>
void launch_d(const SharedPlan& pl, int dtype, int out_dtype, int bs, hipStream_t st) {
    const dim3 grid((unsigned)pl.a.items);   // one workgroup per item
    if (dtype == PAGED_KV_F16) {
        if (bs == 32) launch_items<D, DT_F16, 32>(pl, grid, st);
        else launch_items<D, DT_F16, 16>(pl, grid, st);
    } else {
        if (bs == 32) launch_items<D, DT_BF16, 32>(pl, grid, st);
        else launch_items<D, DT_BF16, 16>(pl, grid, st);
    }
    const dim3 mgrid((unsigned)pl.a.num_kv_heads, (unsigned)pl.a.num_seqs);
    const int outs = pl.a.group * D;
    const dim3 mblock((unsigned)std::min(1024, ((outs + kMergeOut - 1) / kMergeOut + 63) / 64 * 64));
    if (pl.a.max_parts <= 2) launch_merge<D, 2>(pl, out_dtype, mgrid, mblock, st);
    else if (pl.a.max_parts <= 4) launch_merge<D, 4>(pl, out_dtype, mgrid, mblock, st);
    else launch_merge<D, 8>(pl, out_dtype, mgrid, mblock, st);
}

// Default partition size: the largest of 4096 tokens (or the longest context, rounded up
// to 512), 2048, 1024, 512 at which the launch still has about four workgroups per compute
// unit (prefix items, plus tail items counted at the tails' longest possible length).
// Fewer, longer partitions mean fewer partial states to store and merge; on 32 prompts
// x 8 samples (2,048 shared tokens, tails up to 520) the launch pair took 153 / 130 / 121
// / 119 us at 512 / 1024 / 2048 / 4096 tokens.
int32_t default_partition_tokens(int64_t num_seqs, int64_t hkv, int64_t num_groups,
                                 int32_t max_shared, int32_t max_ctx) {
    const int64_t want = 4 * (int64_t)pkv::device_shape().compute_units;
    int32_t pt = std::min(4096, (max_ctx + 511) / 512 * 512);
    while (pt > 512) {
        const int64_t items = num_groups * hkv * ((max_shared + pt - 1) / pt) +
                              num_seqs * hkv * ((max_ctx - max_shared + pt - 1) / pt);
        if (items >= want) break;
        pt = std::max(512, pt / 2 / kTile * kTile);
    }
    return std::max(pt, (int32_t)kTile);
}

paged_kv_status plan_shared(SharedPlan& pl, const paged_kv_pool_desc* desc, int32_t num_seqs,
                            int32_t hq, int32_t max_ctx, int32_t num_groups, int32_t max_group,
                            int32_t max_shared, int32_t part_tokens) {
    if (!pkv::kernel_desc(desc, true)) return PAGED_KV_ERR_INVALID_ARG;
    if (num_seqs < 0 || hq < 1 || hq % desc->num_kv_heads) {
        pkv::set_error("num_seqs %d < 0, or num_q_heads %d not a positive multiple of %d",
                       num_seqs, hq, desc->num_kv_heads);
        return PAGED_KV_ERR_INVALID_ARG;
    }
    const int group = hq / desc->num_kv_heads;
    if (desc->dtype == PAGED_KV_F32 || group < 2 || desc->block_size < 16) {
        pkv::set_error("shared-prefix decode needs an fp16/bf16 pool, >= 2 query heads per KV "
                       "head and 16- or 32-token blocks");
        return PAGED_KV_ERR_UNSUPPORTED;
    }
    if (max_ctx < 1 || num_groups < (num_seqs > 0 ? 1 : 0) || max_group < 1 || max_shared < 0 ||
        max_shared > max_ctx) {
        pkv::set_error("need max_context_len >= 1, num_groups >= 1, max_group >= 1 and "
                       "0 <= max_shared_tokens <= max_context_len");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    pl.nb = n_blocks_for(max_group, group);
    if (pl.nb == 0) {
        pkv::set_error("max_group (%d) x query heads per KV head (%d) must be at most 64",
                       max_group, group);
        return PAGED_KV_ERR_UNSUPPORTED;
    }
    // One item serves the whole group (up to 4 N-blocks).  Serving 32 query slots as two
    // 16-slot items that read the same shared tiles (three waves per SIMD instead of two)
    // measured slower on the parallel-sampling workload: 148 against 136 us.
    if (part_tokens == 0)
        part_tokens = default_partition_tokens(num_seqs, desc->num_kv_heads, num_groups, max_shared, max_ctx);
    if (part_tokens < 0 || part_tokens % kTile) {
        pkv::set_error("partition_tokens %d must be 0 or a positive multiple of %d", part_tokens, kTile);
        return PAGED_KV_ERR_INVALID_ARG;
    }
    SharedArgs& a = pl.a;
    a = SharedArgs{};
    a.num_seqs = num_seqs;
    a.num_groups = num_groups;
    a.max_group = max_group;
    a.num_q_heads = hq;
    a.num_kv_heads = desc->num_kv_heads;
    a.group = group;
    a.num_blocks = desc->num_blocks;
    a.max_context_len = max_ctx;
    a.partition_tokens = part_tokens;
    a.max_shared = max_shared;
    a.block_size = desc->block_size;
    a.prefix_parts = (max_shared + part_tokens - 1) / part_tokens;
    a.tail_parts = (max_ctx + part_tokens - 1) / part_tokens;
    a.max_parts = a.prefix_parts + a.tail_parts;
    a.members_per_item = std::max(1, 16 * pl.nb / group);
    a.chunks = (max_group + a.members_per_item - 1) / a.members_per_item;
    a.prefix_items = (int64_t)num_groups * desc->num_kv_heads * a.prefix_parts * a.chunks;
    a.items = a.prefix_items + (int64_t)num_seqs * desc->num_kv_heads * a.tail_parts;
    if (a.items > INT32_MAX || num_seqs > 65535) {
        pkv::set_error("batch too large for one launch");
        return PAGED_KV_ERR_UNSUPPORTED;
    }
    pl.ws_bytes = shared_workspace(num_seqs, hq, desc->head_dim, a.max_parts);
    return PAGED_KV_OK;
}

}  // namespace

extern "C" {

size_t paged_attention_shared_prefix_workspace_bytes(const paged_kv_pool_desc* desc,
                                                     int32_t num_seqs, int32_t num_q_heads,
                                                     int32_t max_context_len, int32_t num_groups,
                                                     int32_t max_group, int32_t max_shared_tokens,
                                                     int32_t partition_tokens) {
    SharedPlan pl;
    if (plan_shared(pl, desc, num_seqs, num_q_heads, max_context_len, num_groups, max_group,
                    max_shared_tokens, partition_tokens) != PAGED_KV_OK)
        return 0;
    return pl.ws_bytes;
}

paged_kv_status paged_attention_decode_shared_prefix(
        const paged_kv_pool_desc* desc, void* out, int32_t out_dtype, const void* q,
        const void* k_pool, const void* v_pool, const int32_t* block_tables,
        int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
        int32_t num_q_heads, int32_t max_context_len, float scale, const int32_t* group_start,
        const int32_t* shared_tokens, int32_t num_groups, int32_t max_group,
        int32_t max_shared_tokens, int32_t partition_tokens, void* workspace,
        size_t workspace_bytes, void* stream) {
    pkv::clear_error();
    SharedPlan pl;
    paged_kv_status st = plan_shared(pl, desc, num_seqs, num_q_heads, max_context_len, num_groups,
                                     max_group, max_shared_tokens, partition_tokens);
    if (st != PAGED_KV_OK) return st;
    if (out_dtype != desc->dtype && out_dtype != PAGED_KV_F32) {
        pkv::set_error("out_dtype must be the pool dtype or fp32");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    if ((int64_t)max_blocks_per_seq * desc->block_size < max_context_len) {
        pkv::set_error("max_blocks_per_seq %d cannot hold max_context_len %d", max_blocks_per_seq,
                       max_context_len);
        return PAGED_KV_ERR_INVALID_ARG;
    }
    if (num_seqs == 0) return PAGED_KV_OK;
    if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !group_start ||
        !shared_tokens) {
        pkv::set_error("null pointer argument");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    if (!workspace || workspace_bytes < pl.ws_bytes) {
        pkv::set_error("workspace of %zu bytes needed (%zu given)", pl.ws_bytes, workspace_bytes);
        return PAGED_KV_ERR_BUFFER_TOO_SMALL;
    }
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_pool) |
         reinterpret_cast<uintptr_t>(v_pool) | reinterpret_cast<uintptr_t>(workspace)) & 15) {
        pkv::set_error("q, pools and workspace must be 16-byte aligned");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    SharedArgs& a = pl.a;
    a.out = out;
    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.group_start = group_start;
    a.shared_tokens = shared_tokens;
    const size_t rows = (size_t)num_seqs * num_q_heads * a.max_parts;
    char* ws = static_cast<char*>(workspace);
    a.seq_desc = reinterpret_cast<i32x4*>(ws);
    ws += desc_region(num_seqs);
    a.ws_m = reinterpret_cast<float*>(ws);
    a.ws_l = reinterpret_cast<float*>(ws + align256(rows * 4));
    a.ws_acc = reinterpret_cast<float*>(ws + 2 * align256(rows * 4));
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.scale_log2 = scale * kLog2e;
    hipStream_t sm = reinterpret_cast<hipStream_t>(stream);
    switch (desc->head_dim) {
        case 64: launch_d<64>(pl, desc->dtype, out_dtype, desc->block_size, sm); break;
        case 256: launch_d<256>(pl, desc->dtype, out_dtype, desc->block_size, sm); break;
        default: launch_d<128>(pl, desc->dtype, out_dtype, desc->block_size, sm); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        pkv::set_error("shared-prefix attention launch failed: %s", hipGetErrorString(e));
        return PAGED_KV_ERR_HIP;
    }
    return PAGED_KV_OK;
}

}  // extern "C"
