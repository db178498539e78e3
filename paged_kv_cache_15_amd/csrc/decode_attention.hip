// Paged decode attention for gfx950: split-K partition kernels and the merge kernel.
//
// What is computed (deepsonar "PagedAttention de vLLM …" §2.2 and §2.6; chester-dev
// "vLLM transforme la mémoire GPU …", PagedAttention section): one query per head per
// sequence attends over that sequence's tokens, whose K/V blocks are gathered from
// anywhere in the pool through the block table.  How (deeplearn.tn "PagedAttention :
// comment optimiser la mémoire GPU …", PagedAttention vs. FlashAttention): tiles of K
// and V are brought on chip and reduced with an incremental softmax, so nothing of
// size context x heads goes back to HBM.
//
// Work decomposition: one workgroup of 4 wave64s per (sequence, KV head, partition of
// `partition_tokens` tokens).  Wave w takes the partition's 16-token tiles w, w+4,
// w+8, ..., keeps its own running max / sum / weighted-V state, and the four
// states are merged in LDS in fixed wave order.  A sequence that fits one partition
// writes its output directly; longer ones leave (max, sum, weighted V) per partition
// in the workspace and attn_reduce_kernel merges them (log-sum-exp, partition order).
// Every summation order depends only on logical token positions, never on where a
// block sits in the pool, so placement and sharing leave results bit-identical.
//
// Two partition kernels:
//   attn_mfma_kernel  fp16/bf16 with >= 2 query heads per KV head: the group's
//     queries form the N side of MFMA tiles, so the scores (16 tokens x group) and
//     the value product (head_dim x group) are dense contractions on the matrix cores.
//   attn_valu_kernel  one query head per workgroup (a group of 1, or fp32): q.k is a
//     GEMV, done on the vector ALUs with cross-lane reductions.
// Scores are kept in the base-2 domain: x = (scale * log2 e) * q.k, weights 2^(x - m).
//
// Pool layout (X = 16 bytes / element size, BS = block size):
//   K [block][kv_head][head_dim / X][BS][X]   V [block][kv_head][head_dim][BS]
// except that a block of 32 tokens is stored as two 16-token sub-blocks one after the
// other (K [block][kv_head][2][head_dim / X][16][X], V [block][kv_head][2][head_dim][16]),
// so a (block, KV head) region is BS * head_dim contiguous elements and a 16-token tile
// is always 16 * head_dim contiguous elements when BS >= 16: every operand load
// instruction reads one contiguous run across its 64 lanes.  With BS = 1 a tile gathers
// 16 blocks, each lane loading from its own token's block, and V (stored token-major at
// that size) is turned into the V^T operand through LDS.

#include <mutex>

#include "attention_common.h"
#include "attention_host.h"

namespace {

using namespace pkv_dev;

struct PartitionArgs {
    void* out;
    const void* q;
    const void* k_pool;
    const void* v_pool;
    const int32_t* block_tables;
    const int32_t* context_lens;
    float* ws_m;
    float* ws_l;
    float* ws_acc;
    int32_t max_blocks_per_seq;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;
    int32_t num_blocks;
    int32_t max_context_len;
    int32_t partition_tokens;
    int32_t max_parts;
    float scale_log2;  // scale * log2(e)
    // Fused decode step (paged_attention_decode_append, MFMA kernel only): the new token
    // of sequence s (rows new_k/new_v [num_seqs][num_kv_heads][head_dim]) is written to
    // pool slot slots[s] by the workgroup that later reads it, and the workgroup that
    // finishes a (sequence, KV head) last merges its partitions (counters: one int32 per
    // (sequence, KV head), zero on entry and left zero).
    const void* new_k;
    const void* new_v;
    const int32_t* slots;
    int32_t* counters;
    int64_t num_slots;
};

// One step of the partitions' log-sum-exp merge: state (M, l, acc) takes in a
// partition's (m_i, l_i, acc_i).  Written with explicit fused multiply-adds so that
// every kernel that merges (the merge kernel, the fused decode step) rounds alike.
__device__ __forceinline__ void lse_fold(float& M, float& l, float& acc, float mi, float li, float ai) {
    const float mn = fmaxf(M, mi);
    const float sc = exp2_fast(M - mn), w = exp2_fast(mi - mn);
    l = fmaf(w, li, l * sc);
    acc = fmaf(w, ai, acc * sc);
    M = mn;
}

// Final write of a workgroup's merged state for query head h (index into the group gq):
// normalised output for a one-partition sequence, raw state for the merge otherwise.
template <int D, int OUT_DT>
__device__ __forceinline__ void write_partition_result(const PartitionArgs& a, int s, int h,
                                                       int p, int npart, int d, float m, float l,
                                                       float acc, bool bad) {
    if (bad) {
        m = NAN;
        l = NAN;
        acc = NAN;
    }
    if (npart == 1) {
        store_out<OUT_DT>(a.out, ((int64_t)s * a.num_q_heads + h) * D + d, acc / l);
    } else {
        const int64_t row = ((int64_t)s * a.num_q_heads + h) * a.max_parts + p;
        a.ws_acc[row * D + d] = acc;
        if (d == 0) {
            a.ws_m[row] = m;
            a.ws_l[row] = l;
        }
    }
}

// ---------------------------------------------------------------------------------
// MFMA partition kernel: fp16/bf16, group of 2..16 query heads per KV head.
//
// Per block of 16 tokens a wave computes S^T = K . Q^T with v_mfma_f32_16x16x32
// (M = 16 tokens, N = 16 query-head slots, K = 32 dims per instruction; D/32 of
// them), then O^T += V^T . P^T with v_mfma_f32_16x16x16 (M = 16 dims per instruction,
// D/16 of them; N = head slots; K = the 16 tokens), P entering as a 16-bit head and a
// 16-bit remainder (two MFMAs per tile).  Lane l works on head slot l % 16
// and token quad l / 16, which is exactly the layout the score tile comes out in and
// the layout the value product wants its B operand in, so P never leaves registers.
// ---------------------------------------------------------------------------------
// Fused decode step: the new token's K/V row of (sequence s, KV head g) into its pool
// slot, in the layout reshape_and_cache writes (threads 0 .. D/X - 1, one 16-byte chunk
// each); a slot outside [0, num_slots) is skipped.
template <int D, int BS>
__device__ __forceinline__ void write_new_token(const PartitionArgs& a, int s, int g) {
    constexpr int X = 8;                      // 16-bit elements per 16-byte chunk
    constexpr int TB = BS < kTile ? BS : kTile;
    const int c = threadIdx.x;
    if (c >= D / X) return;
    const int32_t slot = a.slots[s];
    if (slot < 0 || (int64_t)slot >= a.num_slots) return;
    const int64_t row = ((int64_t)s * a.num_kv_heads + g) * D + c * X;
    const i32x4 kc = *reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(a.new_k) + row);
    const i32x4 vc = *reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(a.new_v) + row);
    const int64_t blk = slot / BS;
    const int32_t sub = (slot % BS) / TB, off = slot % TB;
    const int64_t region = (blk * a.num_kv_heads + g) * (BS / TB) + sub;
    uint16_t* kdst = static_cast<uint16_t*>(const_cast<void*>(a.k_pool)) + ((region * (D / X) + c) * TB + off) * X;
    *reinterpret_cast<i32x4*>(kdst) = kc;
    uint16_t* vdst = static_cast<uint16_t*>(const_cast<void*>(a.v_pool)) + (region * D + (int64_t)c * X) * TB + off;
    if constexpr (BS == 1) {
        *reinterpret_cast<i32x4*>(vdst) = vc;
    } else {
#pragma unroll
        for (int e = 0; e < X; ++e) vdst[e * TB] = (uint16_t)((uint32_t)vc[e / 2] >> (16 * (e % 2)));
    }
}

// Waves per workgroup.  Eight measured slower for the small-batch fused decode step:
// its tile loop already moves the launch's K/V at the HBM rate (shorter per-wave chains
// of tiles save nothing there), while the per-workgroup start and merge costs grow.
template <bool FUSE, int D>
constexpr int mfma_partition_waves() { return kWaves; }

// (Block size 1 at head_dim 128 needs more than a third of the register file for its LDS
// round trips: two waves per SIMD there.)
template <int D, int DT, int OUT_DT, int BS, bool FUSE>
__global__ __launch_bounds__((mfma_partition_waves<FUSE, D>() * 64))
__attribute__((amdgpu_waves_per_eu(BS == 1 && D == 128 ? 2 : mfma_waves_per_simd<D, false>())))
void attn_mfma_kernel(PartitionArgs a) {
    constexpr int NW = mfma_partition_waves<FUSE, D>();
    constexpr int KI = D / 32;   // QK MFMAs (and 16-byte K loads per lane) per tile
    constexpr int MT = D / 16;   // PV MFMA pairs (and 8-byte V loads per lane) per tile
    constexpr int TILE = BS * D;  // elements of one (block, KV head) region
    constexpr int TPB = BS >= kTile ? BS / kTile : 1;   // tiles per block
    constexpr int LDW = D + 8;    // block size 1: LDS row of one token's values
    using kvec = typename std::conditional<DT == DT_BF16, bf16x8, f16x8>::type;
    using vbuf = typename std::conditional<BS == 1, i32x4[KI], i32x2[MT]>::type;
    // Block size 1: each wave's K and V rows during the tile loop, then (all waves past
    // it) the wave merge's values; other block sizes keep the merge values apart.
    __shared__ __attribute__((aligned(16))) uint16_t s_rows[BS == 1 ? 2 * NW * kTile * LDW : 1];
    __shared__ __attribute__((aligned(16))) float s_merge[BS == 1 ? 4 : NW * 16 * (D + 4)];
    static_assert(BS != 1 || 2 * NW * kTile * LDW * 2 >= NW * 16 * (D + 4) * 4, "merge fits the rows");
    uint16_t* const s_vt = s_rows;
    uint16_t* const s_kt = s_rows + NW * kTile * LDW;
    float* const sm_acc = BS == 1 ? reinterpret_cast<float*>(s_rows) : s_merge;

    const int s = blockIdx.x / a.num_kv_heads, g = blockIdx.x - s * a.num_kv_heads;
    const int p = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int gq = lane & 15, quad = lane >> 4;
    const int ctx = a.context_lens[s];
    const bool bad_len = ctx < 1 || ctx > a.max_context_len;
    const int start = p * a.partition_tokens;
    const int npart = bad_len ? 1 : (ctx + a.partition_tokens - 1) / a.partition_tokens;
    if (FUSE && bad_len) {
        // nothing reads this sequence's blocks: the write only has to happen
        if (p == 0) write_new_token<D, BS>(a, s, g);
    }
    if (bad_len) {
        if (p == 0) {
            for (int i = threadIdx.x; i < a.group * D; i += blockDim.x)
                store_out<OUT_DT>(a.out, ((int64_t)s * a.num_q_heads + g * a.group + i / D) * D + i % D, NAN);
        }
        return;
    }
    if (start >= ctx) return;
    const int end = min(start + a.partition_tokens, ctx);
    const int blk_begin = start / kTile, blk_end = (end + kTile - 1) / kTile;   // tiles
    const int32_t* trow = a.block_tables + (int64_t)s * a.max_blocks_per_seq;

    // Query operand: lane holds q[head gq][32*kk + 8*quad .. +8] for each kk.
    kvec qop[KI];
    {
        const uint16_t* qh = static_cast<const uint16_t*>(a.q) +
                             ((int64_t)s * a.num_q_heads + g * a.group + gq) * D + 8 * quad;
#pragma unroll
        for (int kk = 0; kk < KI; ++kk) {
            i32x4 v = {0, 0, 0, 0};
            if (gq < a.group) v = *reinterpret_cast<const i32x4*>(qh + 32 * kk);
            qop[kk] = __builtin_bit_cast(kvec, v);
        }
    }

    const uint16_t* kbase = static_cast<const uint16_t*>(a.k_pool) + (int64_t)g * (BS == 1 ? D : TILE);
    const uint16_t* vbase = static_cast<const uint16_t*>(a.v_pool) + (int64_t)g * (BS == 1 ? D : TILE);
    const int64_t blk_stride = (int64_t)a.num_kv_heads * TILE;
    const int voff = gq * 4 + quad;   // 8-byte unit of row gq, tokens 4*quad.. of a V^T tile
    uint16_t* vrows = s_vt + w * kTile * LDW;
    uint16_t* krows = s_kt + w * kTile * LDW;

    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m = kNegInf, lsum = 0.f;
    bool bad_block = false;

    i32x4 kA[KI], kB[KI];
    vbuf vA, vB;
    int id_v = 0;    // block size >= 16: lane i holds the block of the wave's i-th tile

    // K tile (block size >= 16): load kk of lane l is 16-byte chunk 4*kk + l/16 of token
    // l%16 (block size 16: bytes [1024*kk + 16*l, +16), each load instruction reads 1 KiB
    // contiguous).  V^T tile: load mt of lane l is row 16*mt + l%16, tokens 4*(l/16)..+3.
    // Block size 1: whole rows, load i of lane l is chunk l % (D / 8) of token
    // (512 / D) i + l / (D / 8), for K and V alike.
    // Block size 1: lane l's id is that of token l % 16 of the tile (tokens at or past ctx
    // take token ctx - 1's), read with a vector load one tile ahead, before the current
    // tile's rows, so that waiting for the ids never waits for those rows.
    int32_t id_next = 0;
    auto fetch_ids = [&](int b) __attribute__((always_inline)) {
        return trow[min(kTile * b + (lane & 15), ctx - 1)];
    };
    auto load = [&](int idx, int b, i32x4 (&kr)[KI], vbuf& vr) __attribute__((always_inline)) {
        if constexpr (BS == 1) {
            const int32_t raw = id_next;                       // tile b's ids
            id_next = fetch_ids(min(b + NW, blk_end - 1));     // the wave's next tile
            __builtin_amdgcn_sched_barrier(0);
            const bool oob = (uint32_t)raw >= (uint32_t)a.num_blocks;
            if (__ballot(oob)) bad_block = true;
            const int32_t idv = oob ? 0 : raw;
#pragma unroll
            for (int i = 0; i < KI; ++i) {
                const int64_t off = load_id_bs1<D>(idv, i, lane) * blk_stride;
                kr[i] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(kbase + off) + lane % (D / 8));
                vr[i] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(vbase + off) + lane % (D / 8));
            }
        } else {
            const int32_t bid = __builtin_amdgcn_readlane(id_v, idx);
            const int64_t sub = (b & (TPB - 1)) * (kTile * D);   // 16-token sub-block
            const i32x4* kt = reinterpret_cast<const i32x4*>(kbase + bid * blk_stride + sub) + lane;
            const i32x2* vt = reinterpret_cast<const i32x2*>(vbase + bid * blk_stride + sub) + voff;
#pragma unroll
            for (int kk = 0; kk < KI; ++kk) kr[kk] = __builtin_nontemporal_load(kt + kk * 64);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) vr[mt] = __builtin_nontemporal_load(vt + mt * 64);
        }
    };

    auto compute = [&](int b, i32x4 (&kr)[KI], vbuf& vin) __attribute__((always_inline)) {
        i32x2 vr[MT];
        if constexpr (BS == 1) {
            // K back in the score product's operand layout, V transposed
            lds_put_whole_rows<D, KI>(krows, LDW, lane, kr);
            lds_put_whole_rows<D, KI>(vrows, LDW, lane, vin);
#pragma unroll
            for (int kk = 0; kk < KI; ++kk)
                kr[kk] = *reinterpret_cast<const i32x4*>(krows + (lane & 15) * LDW + 32 * kk + 8 * (lane >> 4));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                uint32_t e[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) e[j] = vrows[(4 * quad + j) * LDW + 16 * mt + gq];
                vr[mt][0] = (int)(e[0] | e[1] << 16);
                vr[mt][1] = (int)(e[2] | e[3] << 16);
            }
        } else {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) vr[mt] = vin[mt];
        }
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KI; ++kk) {
            if constexpr (DT == DT_BF16)
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[kk]),
                                                             qop[kk], sc, 0, 0, 0);
            else
                sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, kr[kk]),
                                                            qop[kk], sc, 0, 0, 0);
        }
        const int tok0 = b * kTile + 4 * quad;  // this lane's 4 tokens: tok0 .. tok0+3
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = (tok0 + j < end) ? sc[j] * a.scale_log2 : kNegInf;
        // Lazy rescaling: the reference max m only moves when a score exceeds it by more
        // than kRescaleSlack (weights stay <= 2^kRescaleSlack); the softmax is the same
        // for any reference, so most blocks skip the cross-lane max and the rescale.
        const float xm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        if (__ballot(xm > m + kRescaleSlack)) {
            const float mnew = fmaxf(m, max_across_quads(xm));
            const float alpha = exp2_fast(m - mnew);
            lsum *= alpha;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
            m = mnew;
        }
        // The weights enter the value product as 16-bit MFMA operands.  One 16-bit
        // rounding of p costs 2^-9 relative (bf16), which short contexts with spread-out
        // values turn into ~1e-3 output error; so p is split into a 16-bit head and a
        // 16-bit remainder (p = hi + lo to ~2^-17) and both are multiplied in.
        s16x4 phi, plo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float pf = exp2_fast(x[j] - m);
            const uint16_t hi = f32_to_bits16<DT>(pf);
            const uint16_t lo = f32_to_bits16<DT>(pf - bits_to_f32<DT>(hi));
            phi[j] = (short)hi;
            plo[j] = (short)lo;
            lsum += pf;
        }
        if (b * kTile + kTile > end) {
            // tail block: slots past the context may hold anything (NaN included);
            // their weight is 0 but 0 * NaN is not, so clear those value elements
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                uint32_t lo = (uint32_t)vr[mt][0], hi = (uint32_t)vr[mt][1];
                if (tok0 + 0 >= end) lo &= 0xFFFF0000u;
                if (tok0 + 1 >= end) lo &= 0x0000FFFFu;
                if (tok0 + 2 >= end) hi &= 0xFFFF0000u;
                if (tok0 + 3 >= end) hi &= 0x0000FFFFu;
                vr[mt][0] = (int)lo;
                vr[mt][1] = (int)hi;
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if constexpr (DT == DT_BF16) {
                const s16x4 va = __builtin_bit_cast(s16x4, vr[mt]);
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, phi, acc[mt], 0, 0, 0);
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, plo, acc[mt], 0, 0, 0);
            } else {
                const f16x4 va = __builtin_bit_cast(f16x4, vr[mt]);
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, __builtin_bit_cast(f16x4, phi),
                                                               acc[mt], 0, 0, 0);
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, __builtin_bit_cast(f16x4, plo),
                                                               acc[mt], 0, 0, 0);
            }
        }
    };

    // Wave w takes the partition's blocks w, w+4, w+8, ...; lane i holds the id of the
    // wave's i-th block (windows of 64).  Software pipeline, two register sets: the
    // next block's loads are in flight while the current one is computed.  Every path
    // through the loop issues the same loads, so the compiler waits for exactly the
    // current block's loads and never drains the prefetch.
    const int nblk = blk_end - blk_begin;
    const int n_w = nblk > w ? (nblk - w + NW - 1) / NW : 0;
    // the first window's block ids are read before the fused write, so that both wait
    // out the same memory round trips
    int32_t id_first = 0;
    if constexpr (BS != 1)
        if (lane < min(64, n_w)) id_first = trow[(blk_begin + w + NW * lane) / TPB];
    if constexpr (FUSE) {
        // The new token (position ctx - 1) lies in the last partition: that workgroup
        // writes it before any of its waves loads a tile, and its own loads then see it
        // (the stores are complete, and L1 holds nothing of that block yet).
        if (p == npart - 1) {
            write_new_token<D, BS>(a, s, g);
            wait_memory_done();
            __syncthreads();
        }
    }
    if constexpr (BS == 1)
        if (n_w > 0) id_next = fetch_ids(blk_begin + w);
    for (int base = 0; base < n_w; base += 64) {
        const int cnt = min(64, n_w - base);
        const int b0 = blk_begin + w + NW * base;
        if constexpr (BS != 1) {
            id_v = base == 0 ? id_first : 0;
            if (base > 0 && lane < cnt) id_v = trow[(b0 + NW * lane) / TPB];
            const bool id_ok = (uint32_t)id_v < (uint32_t)a.num_blocks;
            if (__ballot(lane < cnt && !id_ok)) bad_block = true;
            id_v = id_ok ? id_v : 0;
        }
        load(0, b0, kA, vA);
        int i = 0;
        for (; i + 2 < cnt; i += 2) {
            load(i + 1, b0 + NW * (i + 1), kB, vB);
            compute(b0 + NW * i, kA, vA);
            load(i + 2, b0 + NW * (i + 2), kA, vA);
            compute(b0 + NW * (i + 1), kB, vB);
        }
        if (i + 1 < cnt) {
            load(i + 1, b0 + NW * (i + 1), kB, vB);
            compute(b0 + NW * i, kA, vA);
            compute(b0 + NW * (i + 1), kB, vB);
        } else {
            compute(b0 + NW * i, kA, vA);
        }
    }

    // ---- merge the four waves' states (fixed order) ----
    // Each wave puts its row maxima, sums and raw values in LDS; after one barrier wave w
    // folds value blocks w*MB .. w*MB + MB - 1 of every row over the waves in order (the
    // first scaled, the rest by fused multiply-adds), so that the four waves share the
    // fold and no wave waits on another's read-modify-write.
    constexpr int MB = MT / NW;
    static_assert(MT % NW == 0, "value blocks split evenly over the waves");
    __shared__ float sm_m[NW][16];
    __shared__ float sm_l[NW][16];
    const float lw = sum_across_quads(lsum);
    if (lane < 16) {
        sm_m[w][lane] = m;
        sm_l[w][lane] = lw;
    }
    float* const my_rows = sm_acc + (w * 16 + gq) * (D + 4) + 4 * quad;
    if constexpr (BS == 1) __syncthreads();   // every wave is past its K/V rows
    if (gq < a.group) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<f32x4*>(my_rows + 16 * mt) = acc[mt];
    }
    const bool any_bad = __syncthreads_or(bad_block);
    // row gq over the waves: the common maximum, each wave's scale, the summed weights
    float mw[NW], lwv[NW], fw[NW];
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
        mw[ww] = sm_m[ww][gq];
        lwv[ww] = sm_l[ww][gq];
    }
    float mm = kNegInf;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) mm = fmaxf(mm, mw[ww]);
    float l = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
        fw[ww] = mw[ww] == kNegInf ? 0.f : exp2_fast(mw[ww] - mm);
        if (mw[ww] != kNegInf) l = fmaf(fw[ww], lwv[ww], l);
    }
    if (gq < a.group) {
        const int h = g * a.group + gq;
        const int64_t row = ((int64_t)s * a.num_q_heads + h) * a.max_parts + p;
#pragma unroll
        for (int j = 0; j < MB; ++j) {
            const int d0 = 16 * (w * MB + j) + 4 * quad;
            f32x4 v;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(sm_acc + (ww * 16 + gq) * (D + 4) + d0);
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = ww == 0 ? x[r] * fw[0] : fmaf(fw[ww], x[r], v[r]);
            }
            if (npart == 1) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    store_out<OUT_DT>(a.out, ((int64_t)s * a.num_q_heads + h) * D + d0 + r,
                                      any_bad ? NAN : v[r] / l);
            } else if (FUSE) {
                // partial state for the merge below, possibly read on another XCD: stored
                // through to the device-coherent level
#pragma unroll
                for (int r = 0; r < 4; ++r) put_coherent(a.ws_acc + row * D + d0 + r, any_bad ? NAN : v[r]);
            } else {
                if (any_bad) v = (f32x4){NAN, NAN, NAN, NAN};
                *reinterpret_cast<f32x4*>(a.ws_acc + row * D + d0) = v;
            }
        }
        if (npart > 1 && w == 0 && quad == 0) {
            if (FUSE) {
                put_coherent(a.ws_m + row, any_bad ? NAN : mm);
                put_coherent(a.ws_l + row, any_bad ? NAN : l);
            } else {
                a.ws_m[row] = any_bad ? NAN : mm;
                a.ws_l[row] = any_bad ? NAN : l;
            }
        }
    }
    if constexpr (FUSE) {
        if (npart > 1) {
            // Count this partition in (s, g)'s counter once its state is stored; the
            // workgroup that brings the count to npart merges all partitions in order
            // (as the merge kernel does with one thread group) and resets the counter.
            // Ordering as in the stream-K merge: sc1 stores complete before the
            // agent-scope count, sc1 loads after it, and a compiler fence between.
            __shared__ int s_old;
            wait_memory_done();
            __syncthreads();
            if (threadIdx.x == 0)
                s_old = __hip_atomic_fetch_add(a.counters + (int64_t)s * a.num_kv_heads + g, 1,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            if (s_old != npart - 1) return;
            __atomic_signal_fence(__ATOMIC_ACQUIRE);
            // NO outputs per thread at a time, KB partitions per memory round trip (all
            // their loads in flight together; four when there are no more, else eight),
            // folded in partition order.
            constexpr int NO = 4;
            for (int i0 = threadIdx.x; i0 < a.group * D; i0 += NO * blockDim.x) {
                float M[NO], l[NO], acc[NO];
                bool bad[NO];
                int64_t row[NO];
                int dd[NO];
#pragma unroll
                for (int o = 0; o < NO; ++o) {
                    M[o] = kNegInf;
                    l[o] = acc[o] = 0.f;
                    bad[o] = false;
                    const int i = min(i0 + o * (int)blockDim.x, a.group * D - 1);
                    dd[o] = i % D;
                    row[o] = ((int64_t)s * a.num_q_heads + g * a.group + i / D) * a.max_parts;
                }
                auto fold = [&](auto kb) __attribute__((always_inline)) {
                    constexpr int KB = decltype(kb)::value;
                    for (int p0 = 0; p0 < npart; p0 += KB) {
                        float mv[NO][KB], lv[NO][KB], av[NO][KB];
#pragma unroll
                        for (int o = 0; o < NO; ++o)
#pragma unroll
                            for (int k = 0; k < KB; ++k) {   // past the last partition: re-read it
                                const int64_t r = row[o] + min(p0 + k, npart - 1);
                                mv[o][k] = get_coherent(a.ws_m + r);
                                lv[o][k] = get_coherent(a.ws_l + r);
                                av[o][k] = get_coherent(a.ws_acc + r * D + dd[o]);
                            }
#pragma unroll
                        for (int o = 0; o < NO; ++o)
#pragma unroll
                            for (int k = 0; k < KB; ++k) {
                                if (p0 + k >= npart) break;
                                bad[o] |= mv[o][k] != mv[o][k];
                                lse_fold(M[o], l[o], acc[o], mv[o][k], lv[o][k], av[o][k]);
                            }
                    }
                };
                if (npart <= 4) fold(std::integral_constant<int, 4>{});
                else fold(std::integral_constant<int, 8>{});
#pragma unroll
                for (int o = 0; o < NO; ++o) {
                    const int i = i0 + o * (int)blockDim.x;
                    if (i < a.group * D)
                        store_out<OUT_DT>(a.out, ((int64_t)s * a.num_q_heads + g * a.group + i / D) * D + i % D,
                                          bad[o] ? NAN : acc[o] / l[o]);
                }
            }
            if (threadIdx.x == 0)
                __hip_atomic_store(a.counters + (int64_t)s * a.num_kv_heads + g, 0, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------------------------
// VALU partition kernel: one query head per workgroup (grid.y = query head).
//
// K tile: load i of lane l covers 16-byte chunk 4*i + l/16 of token l % 16, so a lane
// holds D/4 dims of one token; q.k is finished with two cross-lane adds (xor 16, 32).
// V tile (dim-major): load i covers 16 bytes of row (64*i + l) / E (E = element bytes),
// i.e. X consecutive tokens of one dim; the weights of those tokens are fetched from
// the lanes that own them with ds_bpermute.
// ---------------------------------------------------------------------------------
template <int D, int DT, int OUT_DT, int BS>
__global__ __launch_bounds__(kWaves * 64)
__attribute__((amdgpu_waves_per_eu(valu_waves_per_simd<D, DT == DT_F32 ? 4 : 2, false>())))
void attn_valu_kernel(PartitionArgs a) {
    using bits_t = typename std::conditional<DT == DT_F32, uint32_t, uint16_t>::type;
    constexpr int E = sizeof(bits_t);
    constexpr int X = 16 / E;           // elements per 16-byte chunk
    constexpr int NI = kTile * D * E / 1024;  // 16-byte loads per lane per tile (K or V)
    constexpr int TILE = BS * D;
    constexpr int TPB = BS >= kTile ? BS / kTile : 1;
    constexpr int LDW = D + X;
    __shared__ bits_t s_vt[BS == 1 ? kWaves * kTile * LDW : 1];

    const int s = blockIdx.x / a.num_q_heads, h = blockIdx.x - s * a.num_q_heads;
    const int p = blockIdx.y;
    const int g = h / a.group;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ctx = a.context_lens[s];
    const bool bad_len = ctx < 1 || ctx > a.max_context_len;
    const int start = p * a.partition_tokens;
    if (bad_len) {
        if (p == 0)
            for (int i = threadIdx.x; i < D; i += blockDim.x)
                store_out<OUT_DT>(a.out, ((int64_t)s * a.num_q_heads + h) * D + i, NAN);
        return;
    }
    if (start >= ctx) return;
    const int end = min(start + a.partition_tokens, ctx);
    const int npart = (ctx + a.partition_tokens - 1) / a.partition_tokens;
    const int blk_begin = start / kTile, blk_end = (end + kTile - 1) / kTile;   // tiles
    const int32_t* trow = a.block_tables + (int64_t)s * a.max_blocks_per_seq;

    // scaled query in LDS, then the lane's D/4 dims in registers
    __shared__ float sm_q[D];
    {
        const bits_t* qh = static_cast<const bits_t*>(a.q) + ((int64_t)s * a.num_q_heads + h) * D;
        for (int i = threadIdx.x; i < D; i += blockDim.x)
            sm_q[i] = bits_to_f32<DT>(qh[i]) * a.scale_log2;
    }
    __syncthreads();
    const int tok = lane & 15;       // K: token of this lane
    const int kq = lane >> 4;        // K: chunk quad
    const int vpiece = lane % E;     // V: which X-token piece of a row this lane reads
    float qr[NI][X];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int e = 0; e < X; ++e) qr[i][e] = sm_q[(4 * i + kq) * X + e];

    const bits_t* kbase = static_cast<const bits_t*>(a.k_pool) + (int64_t)g * (BS == 1 ? D : TILE);
    const bits_t* vbase = static_cast<const bits_t*>(a.v_pool) + (int64_t)g * (BS == 1 ? D : TILE);
    const int64_t blk_stride = (int64_t)a.num_kv_heads * TILE;
    bits_t* vrows = s_vt + w * kTile * LDW;

    float acc[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) acc[i] = 0.f;
    float m = kNegInf, lsum = 0.f;
    bool bad_block = false;
    i32x4 kA[NI], kB[NI], vA[NI], vB[NI];
    int id_v = 0;

    auto load = [&](int idx, int b, i32x4 (&kr)[NI], i32x4 (&vr)[NI]) __attribute__((always_inline)) {
        if constexpr (BS == 1) {
            bool bad;
            const int32_t bid = lane_block_bs1(trow, b, ctx, a.num_blocks, lane, bad);
            bad_block |= bad;
            const i32x4* kt = reinterpret_cast<const i32x4*>(kbase + bid * blk_stride) + kq;
            const i32x4* vt = reinterpret_cast<const i32x4*>(vbase + bid * blk_stride) + kq;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                kr[i] = __builtin_nontemporal_load(kt + 4 * i);
                vr[i] = __builtin_nontemporal_load(vt + 4 * i);
            }
        } else {
            const int32_t bid = __builtin_amdgcn_readlane(id_v, idx);
            const int64_t sub = (b & (TPB - 1)) * (kTile * D);   // 16-token sub-block
            const i32x4* kt = reinterpret_cast<const i32x4*>(kbase + bid * blk_stride + sub) + lane;
            const i32x4* vt = reinterpret_cast<const i32x4*>(vbase + bid * blk_stride + sub) + lane;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                kr[i] = __builtin_nontemporal_load(kt + i * 64);
                vr[i] = __builtin_nontemporal_load(vt + i * 64);
            }
        }
    };

    auto compute = [&](int b, i32x4 (&kr)[NI], i32x4 (&vin)[NI]) __attribute__((always_inline)) {
        i32x4 vr[NI];
        if constexpr (BS == 1) {
            lds_put_rows<bits_t, NI>(vrows, LDW, lane, vin);
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                bits_t vb[X];
#pragma unroll
                for (int e = 0; e < X; ++e) vb[e] = vrows[(vpiece * X + e) * LDW + (64 * i + lane) / E];
                __builtin_memcpy(&vr[i], vb, 16);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NI; ++i) vr[i] = vin[i];
        }
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            bits_t kb[X];
            __builtin_memcpy(kb, &kr[i], 16);
#pragma unroll
            for (int e = 0; e < X; ++e) part = fmaf(qr[i][e], bits_to_f32<DT>(kb[e]), part);
        }
        const float sc = sum_across_quads(part);
        const int t = b * kTile + tok;
        const float x = t < end ? sc : kNegInf;
        // lazy rescaling, as in the MFMA kernel
        if (__ballot(x > m + kRescaleSlack)) {
            float mb = x;
            mb = fmaxf(mb, __shfl_xor(mb, 1));
            mb = fmaxf(mb, __shfl_xor(mb, 2));
            mb = fmaxf(mb, __shfl_xor(mb, 4));
            mb = fmaxf(mb, __shfl_xor(mb, 8));
            const float mnew = fmaxf(m, mb);
            const float alpha = exp2_fast(m - mnew);
            lsum *= alpha;
#pragma unroll
            for (int i = 0; i < NI; ++i) acc[i] *= alpha;
            m = mnew;
        }
        const float pt = exp2_fast(x - m);
        lsum += pt;
        float pw[X];
#pragma unroll
        for (int e = 0; e < X; ++e) pw[e] = __shfl(pt, vpiece * X + e);
        const int valid = end - b * kTile;   // tokens of this tile inside the partition
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            bits_t vb[X];
            __builtin_memcpy(vb, &vr[i], 16);
            float r = acc[i];
#pragma unroll
            for (int e = 0; e < X; ++e) {
                // slots past the context may hold NaN: select, never multiply by 0
                const float v = (vpiece * X + e < valid) ? bits_to_f32<DT>(vb[e]) : 0.f;
                r = fmaf(pw[e], v, r);
            }
            acc[i] = r;
        }
    };

    // same schedule and pipeline as the MFMA kernel
    const int nblk = blk_end - blk_begin;
    const int n_w = nblk > w ? (nblk - w + kWaves - 1) / kWaves : 0;
    for (int base = 0; base < n_w; base += 64) {
        const int cnt = min(64, n_w - base);
        const int b0 = blk_begin + w + kWaves * base;
        if constexpr (BS != 1) {
            id_v = 0;
            if (lane < cnt) id_v = trow[(b0 + kWaves * lane) / TPB];
            const bool id_ok = (uint32_t)id_v < (uint32_t)a.num_blocks;
            if (__ballot(lane < cnt && !id_ok)) bad_block = true;
            id_v = id_ok ? id_v : 0;
        }
        load(0, b0, kA, vA);
        int i = 0;
        for (; i + 2 < cnt; i += 2) {
            load(i + 1, b0 + kWaves * (i + 1), kB, vB);
            compute(b0 + kWaves * i, kA, vA);
            load(i + 2, b0 + kWaves * (i + 2), kA, vA);
            compute(b0 + kWaves * (i + 1), kB, vB);
        }
        if (i + 1 < cnt) {
            load(i + 1, b0 + kWaves * (i + 1), kB, vB);
            compute(b0 + kWaves * i, kA, vA);
            compute(b0 + kWaves * (i + 1), kB, vB);
        } else {
            compute(b0 + kWaves * i, kA, vA);
        }
    }

    // lane sums: each token's weight sits in its 16-lane row 4 times; take one row
    float lw = lsum;
    lw += __shfl_xor(lw, 1);
    lw += __shfl_xor(lw, 2);
    lw += __shfl_xor(lw, 4);
    lw += __shfl_xor(lw, 8);
    // value rows: the E lanes that share a row hold disjoint token pieces
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        if constexpr (E >= 2) acc[i] += __shfl_xor(acc[i], 1);
        if constexpr (E >= 4) acc[i] += __shfl_xor(acc[i], 2);
    }

    __shared__ float sm_m[kWaves], sm_l[kWaves];
    __shared__ float sm_acc[D];
    if (lane == 0) {
        sm_m[w] = m;
        sm_l[w] = lw;
    }
    const bool any_bad = __syncthreads_or(bad_block);
    float mmax = kNegInf;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) mmax = fmaxf(mmax, sm_m[ww]);
    const float f = (m == kNegInf) ? 0.f : exp2_fast(m - mmax);
    for (int ww = 0; ww < kWaves; ++ww) {
        if (ww == w && vpiece == 0) {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int d = (64 * i + lane) / E;
                const float v = acc[i] * f;
                if (ww == 0) sm_acc[d] = v;
                else sm_acc[d] += v;
            }
        }
        __syncthreads();
    }
    float l = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww)
        if (sm_m[ww] != kNegInf) l += exp2_fast(sm_m[ww] - mmax) * sm_l[ww];
    for (int d = threadIdx.x; d < D; d += blockDim.x)
        write_partition_result<D, OUT_DT>(a, s, h, p, npart, d, mmax, l, sm_acc[d], any_bad);
}

// ---------------------------------------------------------------------------------
// Merge of the partitions of one (sequence, query head): with M the largest partition
// max, out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p, partitions in order.
// ---------------------------------------------------------------------------------
constexpr int kReduceMaxGroups = 8;
// groups of D threads per workgroup: at most 8, and at most 1024 threads
template <int D>
constexpr int reduce_groups_max() { return 1024 / D < kReduceMaxGroups ? 1024 / D : kReduceMaxGroups; }

// PAIRS: the partition states of the stream-K schedule (pkv::StreamLaunch::pm_tiles): two
// rows per partition, the second a cut-off rest (skipped when its m is -inf, which no
// computed piece has), and every sequence has rows (one-partition ones included).
template <int D, int OUT_DT, bool PAIRS>
__global__ __launch_bounds__(D * reduce_groups_max<D>()) void attn_reduce_kernel(
        void* out, const int32_t* context_lens, int32_t num_q_heads, int32_t max_context_len,
        int32_t partition_tokens, int32_t max_parts, const float* ws_m, const float* ws_l,
        const float* ws_acc) {
    // One workgroup per (query head, sequence) of R = blockDim.x / D groups of D threads
    // (one thread per head dim).  Group g folds partitions [g*per, (g+1)*per) in order,
    // eight per memory round trip, by an online log-sum-exp:
    //   M' = max(M, m_i), L' = L 2^(M - M') + l_i 2^(m_i - M'), acc likewise;
    // group 0 then folds the groups' states in group order.
    __shared__ float s_acc[kReduceMaxGroups][D];
    __shared__ float s_ml[kReduceMaxGroups][2];
    __shared__ int s_bad[kReduceMaxGroups];
    const int R = blockDim.x / D, g = threadIdx.x / D, d = threadIdx.x % D;
    const int s = blockIdx.y, h = blockIdx.x;
    const int64_t o = ((int64_t)s * num_q_heads + h) * D + d;
    const int ctx = context_lens[s];
    if (ctx < 1 || ctx > max_context_len) {
        if (g == 0) store_out<OUT_DT>(out, o, NAN);
        return;
    }
    const int parts = (ctx + partition_tokens - 1) / partition_tokens;
    if (!PAIRS && parts == 1) return;   // written by the partition kernel
    const int np = PAIRS ? 2 * parts : parts;   // rows to fold
    const int64_t row = ((int64_t)s * num_q_heads + h) * (PAIRS ? 2 * max_parts : max_parts);
    const int per = (np + R - 1) / R;
    const int i_lo = min(np, g * per), i_hi = min(np, i_lo + per);
    float M = kNegInf, l = 0.f, acc = 0.f;
    bool bad = false;
    for (int i0 = i_lo; i0 < i_hi; i0 += 8) {
        float mv[8], lv[8], av[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {   // slots past the range re-read its last partition
            const int64_t r = row + min(i0 + k, i_hi - 1);
            mv[k] = ws_m[r];
            lv[k] = ws_l[r];
            av[k] = ws_acc[r * D + d];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (i0 + k >= i_hi) break;
            if (PAIRS && mv[k] == kNegInf) continue;
            bad |= mv[k] != mv[k];
            lse_fold(M, l, acc, mv[k], lv[k], av[k]);
        }
    }
    if (R > 1) {
        s_acc[g][d] = acc;
        if (d == 0) {
            s_ml[g][0] = M;
            s_ml[g][1] = l;
            s_bad[g] = bad;
        }
        __syncthreads();
        if (g != 0) return;
        for (int gg = 1; gg < R; ++gg) {   // group 0 has partitions, so M is finite here
            bad |= s_bad[gg] != 0;
            lse_fold(M, l, acc, s_ml[gg][0], s_ml[gg][1], s_acc[gg][d]);   // empty group: weight 0
        }
    }
    store_out<OUT_DT>(out, o, bad ? NAN : acc / l);
}

// ---------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------

// Scratch of paged_attention_decode_static, for callers that cannot allocate: a fixed
// region of merge counters (zero between calls: zeroed once per device, and every call
// leaves the counters it uses at zero) followed by room for partial results.  Each device
// the library runs on holds its own copy until the process ends; calls on one device
// share it, so calls that overlap there race.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
constexpr size_t kStaticCounterBytes = size_t(1) << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

__global__ void zero_words(int32_t* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

struct Plan {
    PartitionArgs a;
    int dtype, out_dtype, head_dim, block_size;
    bool mfma;
    bool streamk;              // stream-K schedule (partition_tokens 0) or fixed partitions
    bool fuse = false;         // fused decode step: cache write + attention + merge in one launch
    bool pm = false;           // fixed partitions' states from the stream-K schedule (use_pm)
    pkv::StreamPlan sp;
    pkv::StreamLaunch sl;
    dim3 grid;
    size_t ws_needed;
    hipStream_t stream;
};

// partition_tokens 0 selects stream-K when the batch fits its limits, else the default
// fixed partition size; workspace sizing and both launches apply the same rule.
bool use_streamk(int32_t part_tokens, int32_t num_seqs) {
    return part_tokens == 0 && num_seqs <= pkv::kStreamMaxSeqs;
}

// The automatic schedule (PAGED_KV_PARTITION_AUTO).  Measured on MI355X with 32-layer
// decode steps of 64 query / 8 KV heads, contexts 256..2048: stream-K took 25-30 us a
// layer for 1-8 sequences and 47.5 for 32, fixed partitions 13.5-19.6 and 43.5 (256
// tokens best up to 4 sequences, 512 from 8); on the 128-sequence GQA workload stream-K
// is the faster one.  Thresholds scale with the device's compute units: stream-K from 64
// tiles per resident wave slot (4 SIMDs per compute unit), 512-token partitions from one
// workgroup per compute unit.
constexpr int64_t kAutoTilesPerSlot = 64;

int32_t auto_partition_tokens(const paged_kv_pool_desc* desc, int32_t num_seqs, int32_t hq,
                              int32_t max_ctx) {
    const int64_t cus = pkv::device_shape().compute_units;
    const bool mfma = desc->dtype != PAGED_KV_F32 && hq / desc->num_kv_heads >= 2;
    const int64_t units = (int64_t)num_seqs * (mfma ? desc->num_kv_heads : hq);
    if (units * ((max_ctx + kTile - 1) / kTile) >= kAutoTilesPerSlot * 4 * cus) return 0;
    return units * ((max_ctx + 511) / 512) >= cus ? 512 : 256;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Bytes at the start of every workspace for the stream-K schedule's merge counters, one
// int32 per (sequence, head unit).  Fixed-partition calls reserve the same prefix and
// never touch it, so calls of either schedule leave the counters at zero.
size_t counter_bytes(const paged_kv_pool_desc* desc, int64_t num_seqs, int64_t hq) {
    const bool mfma = desc->dtype != PAGED_KV_F32 && hq / desc->num_kv_heads >= 2;
    return align256((size_t)num_seqs * (mfma ? desc->num_kv_heads : hq) * sizeof(int32_t));
}

// Fixed partitions: counters | m, l: float[rows] | acc: float[rows][d], rows =
// num_seqs * hq * max_parts (twice that for partition states from the stream-K schedule,
// use_pm).  Nothing when no sequence can need a second partition.
size_t workspace_for(size_t cnt_bytes, int64_t num_seqs, int64_t hq, int64_t d, int64_t max_parts,
                     bool pm = false) {
    if (max_parts <= 1) return 0;
    const size_t rows = (size_t)num_seqs * hq * max_parts * (pm ? 2 : 1);
    return cnt_bytes + 2 * align256(rows * sizeof(float)) + rows * d * sizeof(float);
}

// Fixed partitions of long contexts in large batches: the partitions' states come from
// the stream-K schedule (each wave streams a contiguous run of tiles and stores one state
// per partition piece, pkv::StreamLaunch::pm_tiles) rather than from one workgroup per
// partition, and the merge kernel folds them as usual.  From 8 partitions per sequence
// and 16 (sequence, KV head, partition) items per compute unit, MFMA kernels at 16- and
// 32-token blocks, up to 2048 sequences (the kernel's LDS holds a per-sequence prefix
// beside the pieces).
bool use_pm(const paged_kv_pool_desc* desc, int64_t num_seqs, int32_t hq, int64_t max_parts) {
    const int group = hq / desc->num_kv_heads;
    const bool mfma = desc->dtype != PAGED_KV_F32 && group >= 2 && group <= 16;
    // (the kernel addresses the states with 32-bit byte offsets)
    const bool fits = num_seqs * hq * 2 * max_parts * desc->head_dim * 4 < (int64_t(1) << 31);
    return mfma && fits && desc->block_size >= 16 && num_seqs >= 1 && num_seqs <= 2048 && max_parts >= 8 &&
           num_seqs * desc->num_kv_heads * max_parts >= 16 * (int64_t)pkv::device_shape().compute_units;
}

// Where a call's workspace lives: one caller buffer (counters first, then the partial
// results), or the library's static scratch array (a fixed counter region, then the
// partial results).
struct WsSource {
    char* buf;              // caller workspace, or NULL for the static scratch
    size_t bytes;
    char* static_base;      // this device's address of the static scratch array
};

paged_kv_status make_plan(Plan& pl, const paged_kv_pool_desc* desc, void* out, int32_t out_dtype,
                          const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* tables, int32_t max_blocks, const int32_t* lens,
                          int32_t num_seqs, int32_t hq, int32_t max_ctx, float scale,
                          int32_t part_tokens, const WsSource& src, void* stream,
                          bool need_kv) {
    void* ws = src.buf;
    const size_t ws_bytes = src.bytes;
    if (!pkv::kernel_desc(desc, true)) return PAGED_KV_ERR_INVALID_ARG;
    if (num_seqs < 0 || hq < 1) {
        pkv::set_error("num_seqs %d < 0 or num_q_heads %d < 1", num_seqs, hq);
        return PAGED_KV_ERR_INVALID_ARG;
    }
    if (hq % desc->num_kv_heads) {
        pkv::set_error("num_q_heads %d is not a multiple of num_kv_heads %d", hq, desc->num_kv_heads);
        return PAGED_KV_ERR_INVALID_ARG;
    }
    const int group = hq / desc->num_kv_heads;
    if (group > 16) {
        pkv::set_error("at most 16 query heads per KV head (got %d)", group);
        return PAGED_KV_ERR_UNSUPPORTED;
    }
    if (out_dtype != desc->dtype && out_dtype != PAGED_KV_F32) {
        pkv::set_error("out_dtype must be the pool dtype or fp32");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    if (max_ctx < 1) { pkv::set_error("max_context_len must be >= 1"); return PAGED_KV_ERR_INVALID_ARG; }
    if (part_tokens == PAGED_KV_PARTITION_AUTO) part_tokens = auto_partition_tokens(desc, num_seqs, hq, max_ctx);
    pl.streamk = use_streamk(part_tokens, num_seqs);
    if (part_tokens == 0) part_tokens = pkv::kDefaultPartitionTokens;
    if (part_tokens < 0 || part_tokens % kTile) {
        pkv::set_error("partition_tokens %d must be a positive multiple of %d", part_tokens, kTile);
        return PAGED_KV_ERR_INVALID_ARG;
    }
    if ((int64_t)max_blocks * desc->block_size < max_ctx) {
        pkv::set_error("max_blocks_per_seq %d cannot hold max_context_len %d", max_blocks, max_ctx);
        return PAGED_KV_ERR_INVALID_ARG;
    }
    if (num_seqs > 65535) { pkv::set_error("at most 65535 sequences per launch"); return PAGED_KV_ERR_UNSUPPORTED; }
    const int max_parts = (max_ctx + part_tokens - 1) / part_tokens;
    if (max_parts > 65535) { pkv::set_error("at most 65535 partitions per sequence"); return PAGED_KV_ERR_UNSUPPORTED; }
    if (pl.streamk) {
        bool ok = false;
        pl.sp = pkv::stream_plan(num_seqs, hq, desc->num_kv_heads, desc->dtype, desc->head_dim,
                                 max_ctx, &ok);
        pl.ws_needed = pl.sp.ws_bytes;
    } else {
        pl.pm = use_pm(desc, num_seqs, hq, max_parts);
        if (pl.pm) {
            bool ok = false;
            pl.sp = pkv::stream_plan(num_seqs, hq, desc->num_kv_heads, desc->dtype, desc->head_dim,
                                     max_ctx, &ok);
            pl.pm = ok;
        }
        pl.ws_needed = workspace_for(counter_bytes(desc, num_seqs, hq), num_seqs, hq,
                                     desc->head_dim, max_parts, pl.pm);
    }
    if (num_seqs > 0) {
        if (!out || !lens || (need_kv && (!q || !k_pool || !v_pool || !tables))) {
            pkv::set_error("null pointer argument");
            return PAGED_KV_ERR_INVALID_ARG;
        }
        if (src.static_base) {
            const size_t cnt = counter_bytes(desc, num_seqs, hq);
            if (pl.ws_needed > 0 &&
                (cnt > kStaticCounterBytes || pl.ws_needed - cnt > kStaticScratchBytes - kStaticCounterBytes)) {
                pkv::set_error("the static scratch holds %zu counter bytes and %zu bytes of partial "
                               "results; this call needs %zu and %zu (use paged_attention_decode "
                               "with a workspace)", kStaticCounterBytes,
                               kStaticScratchBytes - kStaticCounterBytes, cnt, pl.ws_needed - cnt);
                return PAGED_KV_ERR_BUFFER_TOO_SMALL;
            }
        } else if (pl.ws_needed > 0 && (!ws || ws_bytes < pl.ws_needed)) {
            pkv::set_error("workspace of %zu bytes needed (%zu given)", pl.ws_needed, ws_bytes);
            return PAGED_KV_ERR_BUFFER_TOO_SMALL;
        }
        if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_pool) |
             reinterpret_cast<uintptr_t>(v_pool) | reinterpret_cast<uintptr_t>(ws)) & 15) {
            pkv::set_error("q, pools and workspace must be 16-byte aligned");
            return PAGED_KV_ERR_INVALID_ARG;
        }
    }
    PartitionArgs& a = pl.a;
    a.out = out;
    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.block_tables = tables;
    a.context_lens = lens;
    const size_t rows = (size_t)num_seqs * hq * max_parts * (pl.pm ? 2 : 1);
    // counters, then the partial results (both schedules lay these out from `data` on)
    int32_t* counters = nullptr;
    char* data = nullptr;
    if (pl.ws_needed) {
        if (src.static_base) {
            counters = reinterpret_cast<int32_t*>(src.static_base);
            data = src.static_base + kStaticCounterBytes;
        } else {
            counters = reinterpret_cast<int32_t*>(ws);
            data = static_cast<char*>(ws) + counter_bytes(desc, num_seqs, hq);
        }
    }
    a.ws_m = pl.ws_needed ? reinterpret_cast<float*>(data) : nullptr;
    a.ws_l = pl.ws_needed ? reinterpret_cast<float*>(data + align256(rows * 4)) : nullptr;
    a.ws_acc = pl.ws_needed ? reinterpret_cast<float*>(data + 2 * align256(rows * 4)) : nullptr;
    a.max_blocks_per_seq = max_blocks;
    a.num_q_heads = hq;
    a.num_kv_heads = desc->num_kv_heads;
    a.group = group;
    a.num_blocks = desc->num_blocks;
    a.max_context_len = max_ctx;
    a.partition_tokens = part_tokens;
    a.max_parts = max_parts;
    a.scale_log2 = scale * kLog2e;
    a.new_k = a.new_v = nullptr;
    a.slots = nullptr;
    a.counters = counters;
    a.num_slots = (int64_t)desc->num_blocks * desc->block_size;
    pl.dtype = desc->dtype;
    pl.out_dtype = out_dtype;
    pl.head_dim = desc->head_dim;
    pl.block_size = desc->block_size;
    pl.mfma = desc->dtype != PAGED_KV_F32 && group >= 2;
    // x: (sequence, head) pairs, y: partition.  All first partitions are dispatched
    // first; the empty high partitions of short sequences come last and exit at once.
    pl.grid = dim3((unsigned)((int64_t)num_seqs * (pl.mfma ? desc->num_kv_heads : hq)),
                   (unsigned)max_parts);
    pl.stream = reinterpret_cast<hipStream_t>(stream);
    pl.sl = pkv::StreamLaunch{out, out_dtype, q, k_pool, v_pool, tables, max_blocks, lens,
                              num_seqs, hq, desc->num_kv_heads, desc->num_blocks, desc->dtype,
                              desc->head_dim, desc->block_size, max_ctx, scale, counters,
                              data};
    if (pl.pm) {
        pl.sl.pm_tiles = part_tokens / kTile;
        pl.sl.pm_max_parts = max_parts;
        pl.sl.pm_m = a.ws_m;
        pl.sl.pm_l = a.ws_l;
        pl.sl.pm_acc = a.ws_acc;
    }
    return PAGED_KV_OK;
}

template <int D, int DT, int OUT, int BS>
void launch_partition_t(const Plan& pl) {
    if constexpr (DT == DT_F32) {
        attn_valu_kernel<D, DT, OUT, BS><<<pl.grid, dim3(kWaves * 64), 0, pl.stream>>>(pl.a);
    } else {
        if (pl.mfma && pl.fuse)
            attn_mfma_kernel<D, DT, OUT, BS, true><<<pl.grid, dim3(mfma_partition_waves<true, D>() * 64), 0,
                                                     pl.stream>>>(pl.a);
        else if (pl.mfma)
            attn_mfma_kernel<D, DT, OUT, BS, false><<<pl.grid, dim3(kWaves * 64), 0, pl.stream>>>(pl.a);
        else attn_valu_kernel<D, DT, OUT, BS><<<pl.grid, dim3(kWaves * 64), 0, pl.stream>>>(pl.a);
    }
}

template <int D, int DT, int BS>
void launch_partition_d(const Plan& pl) {
    if (pl.out_dtype == PAGED_KV_F32) launch_partition_t<D, DT, DT_F32, BS>(pl);
    else launch_partition_t<D, DT, DT, BS>(pl);
}

template <int D, int BS>
void launch_partition_dd(const Plan& pl) {
    switch (pl.dtype) {
        case PAGED_KV_F32: launch_partition_d<D, DT_F32, BS>(pl); break;
        case PAGED_KV_F16: launch_partition_d<D, DT_F16, BS>(pl); break;
        default: launch_partition_d<D, DT_BF16, BS>(pl); break;
    }
}

template <int D>
void launch_partition_b(const Plan& pl) {
    switch (pl.block_size) {
        case 1: launch_partition_dd<D, 1>(pl); break;
        case 32: launch_partition_dd<D, 32>(pl); break;
        default: launch_partition_dd<D, 16>(pl); break;
    }
}

template <int D, int OUT>
void launch_reduce_t(const Plan& pl, int num_seqs) {
    // about 16 partitions per thread group, at most reduce_groups_max<D>() groups
    const int rows = pl.pm ? 2 * pl.a.max_parts : pl.a.max_parts;
    const int groups = std::max(1, std::min(reduce_groups_max<D>(), (rows + 15) / 16));
    if (pl.pm)
        attn_reduce_kernel<D, OUT, true><<<dim3((unsigned)pl.a.num_q_heads, (unsigned)num_seqs),
                                           dim3(D * groups), 0,
                                           pl.stream>>>(pl.a.out, pl.a.context_lens, pl.a.num_q_heads,
                                                        pl.a.max_context_len, pl.a.partition_tokens,
                                                        pl.a.max_parts, pl.a.ws_m, pl.a.ws_l, pl.a.ws_acc);
    else
        attn_reduce_kernel<D, OUT, false><<<dim3((unsigned)pl.a.num_q_heads, (unsigned)num_seqs),
                                            dim3(D * groups), 0,
                                            pl.stream>>>(pl.a.out, pl.a.context_lens, pl.a.num_q_heads,
                                                         pl.a.max_context_len, pl.a.partition_tokens,
                                                         pl.a.max_parts, pl.a.ws_m, pl.a.ws_l, pl.a.ws_acc);
}

template <int D>
void launch_reduce_d(const Plan& pl, int num_seqs) {
    switch (pl.out_dtype) {
        case PAGED_KV_F32: launch_reduce_t<D, DT_F32>(pl, num_seqs); break;
        case PAGED_KV_F16: launch_reduce_t<D, DT_F16>(pl, num_seqs); break;
        default: launch_reduce_t<D, DT_BF16>(pl, num_seqs); break;
    }
}

paged_kv_status launch_status(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        pkv::set_error("%s launch failed: %s", what, hipGetErrorString(e));
        return PAGED_KV_ERR_HIP;
    }
    return PAGED_KV_OK;
}

void launch_partition(const Plan& pl, void* stream) {
    if (pl.streamk || pl.pm) pkv::launch_streamk_partition(pl.sl, pl.sp, stream);
    else if (pl.head_dim == 64) launch_partition_b<64>(pl);
    else if (pl.head_dim == 256) launch_partition_b<256>(pl);
    else launch_partition_b<128>(pl);
}

// Fixed partitions only: the merge kernel (stream-K merges inside its one launch).
void launch_reduce(const Plan& pl, int num_seqs) {
    if (pl.streamk || pl.a.max_parts <= 1) return;
    if (pl.head_dim == 64) launch_reduce_d<64>(pl, num_seqs);
    else if (pl.head_dim == 256) launch_reduce_d<256>(pl, num_seqs);
    else launch_reduce_d<128>(pl, num_seqs);
}

// This device's address of the static scratch array (host code may not use the array's
// name itself: on the host it is only a stand-in for the symbol).  Looked up once per
// device with that device current; `zeroed` tells whether its counters were cleared.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_addr[kMaxDevices];
bool g_scratch_zeroed[kMaxDevices];

paged_kv_status static_scratch(int& dev, char*& base) {
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        pkv::set_error("no usable current HIP device for the static scratch");
        return PAGED_KV_ERR_HIP;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            pkv::set_error("hipGetSymbolAddress of the static scratch failed: %s", hipGetErrorString(e));
            return PAGED_KV_ERR_HIP;
        }
        g_scratch_addr[dev] = static_cast<char*>(p);
    }
    base = g_scratch_addr[dev];
    return PAGED_KV_OK;
}

// Clears the counter region on `stream` the first time a call on this device launches
// (a fill kernel, not a memset, so that it may also be recorded into a graph).
paged_kv_status zero_static_counters(int dev, char* base, hipStream_t stream) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_zeroed[dev]) return PAGED_KV_OK;
    zero_words<<<dim3(256), dim3(256), 0, stream>>>(reinterpret_cast<int32_t*>(base),
                                                    (int64_t)(kStaticCounterBytes / sizeof(int32_t)));
    const paged_kv_status st = launch_status("static scratch clear");
    if (st == PAGED_KV_OK) g_scratch_zeroed[dev] = true;
    return st;
}

}  // namespace

extern "C" {

int32_t paged_attention_auto_partition_tokens(const paged_kv_pool_desc* desc, int32_t num_seqs,
                                              int32_t num_q_heads, int32_t max_context_len) {
    if (!pkv::valid_desc(desc) || num_seqs < 0 || num_q_heads < 1 || max_context_len < 1 ||
        num_q_heads % desc->num_kv_heads)
        return -1;
    return auto_partition_tokens(desc, num_seqs, num_q_heads, max_context_len);
}

size_t paged_attention_workspace_bytes(const paged_kv_pool_desc* desc, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t max_context_len,
                                       int32_t partition_tokens) {
    if (!pkv::valid_desc(desc) || num_seqs < 0 || num_q_heads < 1 || max_context_len < 1 ||
        partition_tokens < PAGED_KV_PARTITION_AUTO || num_q_heads % desc->num_kv_heads)
        return 0;
    if (partition_tokens == PAGED_KV_PARTITION_AUTO)
        partition_tokens = auto_partition_tokens(desc, num_seqs, num_q_heads, max_context_len);
    if (use_streamk(partition_tokens, num_seqs)) {
        bool ok = false;
        pkv::StreamPlan p = pkv::stream_plan(num_seqs, num_q_heads, desc->num_kv_heads, desc->dtype,
                                             desc->head_dim, max_context_len, &ok);
        return ok ? p.ws_bytes : 0;
    }
    if (partition_tokens == 0) partition_tokens = pkv::kDefaultPartitionTokens;
    const int64_t max_parts = (max_context_len + (int64_t)partition_tokens - 1) / partition_tokens;
    bool pm = use_pm(desc, num_seqs, num_q_heads, max_parts);
    if (pm) {
        bool ok = false;
        pkv::stream_plan(num_seqs, num_q_heads, desc->num_kv_heads, desc->dtype, desc->head_dim,
                         max_context_len, &ok);
        pm = ok;
    }
    return workspace_for(counter_bytes(desc, num_seqs, num_q_heads), num_seqs, num_q_heads,
                         desc->head_dim, max_parts, pm);
}

paged_kv_status paged_attention_partition(const paged_kv_pool_desc* desc, void* out,
                                          int32_t out_dtype, const void* q, const void* k_pool,
                                          const void* v_pool, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                                          int32_t num_seqs, int32_t num_q_heads,
                                          int32_t max_context_len, float scale,
                                          int32_t partition_tokens, void* workspace,
                                          size_t workspace_bytes, void* stream) {
    pkv::clear_error();
    Plan pl;
    paged_kv_status st = make_plan(pl, desc, out, out_dtype, q, k_pool, v_pool, block_tables,
                                   max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                                   max_context_len, scale, partition_tokens,
                                   WsSource{static_cast<char*>(workspace), workspace_bytes, nullptr},
                                   stream, true);
    if (st != PAGED_KV_OK || num_seqs == 0) return st;
    launch_partition(pl, stream);
    return launch_status("paged attention partition kernel");
}

paged_kv_status paged_attention_reduce(const paged_kv_pool_desc* desc, void* out, int32_t out_dtype,
                                       const int32_t* context_lens, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t max_context_len,
                                       int32_t partition_tokens, const void* workspace,
                                       size_t workspace_bytes, void* stream) {
    pkv::clear_error();
    Plan pl;
    const int32_t max_blocks = desc ? (max_context_len + desc->block_size - 1) / std::max(1, desc->block_size) : 0;
    paged_kv_status st = make_plan(
        pl, desc, out, out_dtype, nullptr, nullptr, nullptr, nullptr, max_blocks, context_lens,
        num_seqs, num_q_heads, max_context_len, 1.f, partition_tokens,
        WsSource{static_cast<char*>(const_cast<void*>(workspace)), workspace_bytes, nullptr}, stream,
        false);
    if (st != PAGED_KV_OK || num_seqs == 0) return st;
    if (pl.streamk || pl.a.max_parts <= 1) return st;   // nothing to merge in a second launch
    launch_reduce(pl, num_seqs);
    return launch_status("paged attention reduce kernel");
}

paged_kv_status paged_attention_decode(const paged_kv_pool_desc* desc, void* out, int32_t out_dtype,
                                       const void* q, const void* k_pool, const void* v_pool,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t max_context_len, float scale,
                                       int32_t partition_tokens, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    paged_kv_status st = paged_attention_partition(
        desc, out, out_dtype, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens,
        num_seqs, num_q_heads, max_context_len, scale, partition_tokens, workspace,
        workspace_bytes, stream);
    if (st != PAGED_KV_OK) return st;
    return paged_attention_reduce(desc, out, out_dtype, context_lens, num_seqs, num_q_heads,
                                  max_context_len, partition_tokens, workspace, workspace_bytes,
                                  stream);
}

paged_kv_status paged_attention_decode_append(const paged_kv_pool_desc* desc, void* out,
                                              int32_t out_dtype, const void* q, const void* new_k,
                                              const void* new_v, const int32_t* slot_mapping,
                                              void* k_pool, void* v_pool,
                                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                                              const int32_t* context_lens, int32_t num_seqs,
                                              int32_t num_q_heads, int32_t max_context_len,
                                              float scale, int32_t partition_tokens, void* workspace,
                                              size_t workspace_bytes, void* stream) {
    pkv::clear_error();
    Plan pl;
    paged_kv_status st = make_plan(pl, desc, out, out_dtype, q, k_pool, v_pool, block_tables,
                                   max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                                   max_context_len, scale, partition_tokens,
                                   WsSource{static_cast<char*>(workspace), workspace_bytes, nullptr},
                                   stream, true);
    if (st != PAGED_KV_OK || num_seqs == 0) return st;
    if (!new_k || !new_v || !slot_mapping) {
        pkv::set_error("null pointer argument");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    if ((reinterpret_cast<uintptr_t>(new_k) | reinterpret_cast<uintptr_t>(new_v)) & 15) {
        pkv::set_error("new_k and new_v must be 16-byte aligned");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    if (pl.streamk || pl.pm || !pl.mfma) {
        // schedules without a fused kernel: the cache write, then the attention
        const int64_t row = (int64_t)desc->num_kv_heads * desc->head_dim;
        st = reshape_and_cache(desc, new_k, new_v, row, row, k_pool, v_pool, slot_mapping, num_seqs, stream);
        if (st != PAGED_KV_OK) return st;
        launch_partition(pl, stream);
        st = launch_status("paged attention partition kernel");
        if (st != PAGED_KV_OK) return st;
        launch_reduce(pl, num_seqs);
        return launch_status("paged attention reduce kernel");
    }
    pl.fuse = true;
    pl.a.new_k = new_k;
    pl.a.new_v = new_v;
    pl.a.slots = slot_mapping;
    launch_partition(pl, stream);
    return launch_status("fused paged decode step kernel");
}

paged_kv_status paged_attention_decode_static(const paged_kv_pool_desc* desc, void* out,
                                              int32_t out_dtype, const void* q, const void* k_pool,
                                              const void* v_pool, const int32_t* block_tables,
                                              int32_t max_blocks_per_seq,
                                              const int32_t* context_lens, int32_t num_seqs,
                                              int32_t num_q_heads, int32_t max_context_len,
                                              float scale, int32_t partition_tokens, void* stream) {
    pkv::clear_error();
    int dev = -1;
    char* base = nullptr;
    paged_kv_status st = static_scratch(dev, base);
    if (st != PAGED_KV_OK) return st;
    Plan pl;
    st = make_plan(pl, desc, out, out_dtype, q, k_pool, v_pool, block_tables, max_blocks_per_seq,
                   context_lens, num_seqs, num_q_heads, max_context_len, scale, partition_tokens,
                   WsSource{nullptr, 0, base}, stream, true);
    if (st != PAGED_KV_OK || num_seqs == 0) return st;
    st = zero_static_counters(dev, base, pl.stream);
    if (st != PAGED_KV_OK) return st;
    launch_partition(pl, stream);
    st = launch_status("paged attention partition kernel");
    if (st != PAGED_KV_OK) return st;
    launch_reduce(pl, num_seqs);
    return launch_status("paged attention reduce kernel");
}

}  // extern "C"
