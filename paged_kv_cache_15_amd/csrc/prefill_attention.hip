// Paged prefill / chunked-prefill attention for gfx950: causal multi-query attention
// over the block pool.
//
// What is computed (deepsonar "PagedAttention de vLLM …" §2.5: a whole prompt, a chunk
// of a long prompt and the rest of a prompt after a prefix-cache hit are one and the
// same step, since a request only counts its computed tokens; §2.6: this attention
// also reads the blocks through the table): the last n_s tokens of sequence s, already
// written to the pool, are queries; query i sits at position ctx_s - n_s + i and
// attends to keys 0 .. that position.  How (deeplearn.tn "PagedAttention : comment
// optimiser la mémoire GPU …", continuous batching section: prefill is the
// compute-heavy phase; PagedAttention vs. FlashAttention: tiles of K and V stream
// through on-chip memory with an incremental softmax, nothing of size queries x keys
// goes back to HBM).
//
// Work decomposition.  A workgroup of 4 waves takes one KV head g of one sequence and
// a run of TQ query tokens; its rows are (token, query head of g's group) pairs,
// token-major, 64*C rows in all (C column blocks of 16 rows per wave).  The workgroup
// walks the keys 0 .. (largest position among its rows) in pairs of 16-token tiles,
// each pair copied once from the pool into LDS and used by all four waves, with the
// decode kernels' orientation: S^T = K . Q^T (v_mfma_f32_16x16x32, query rows on the N
// side) and O^T += V^T . P^T over the pair (v_mfma_f32_16x16x32 with K = 32 keys; the
// weights come out of the score product already in the B-operand layout).  The causal
// mask is per lane (each lane owns one query row of a block) and only applied to pairs
// that reach past a row's position; the online softmax is base 2 with lazy rescaling,
// tested once per pair for all blocks, and the pairs that need neither the mask nor any
// clearing of slots past the context run a branch-free step.  The query tiles of one
// (sequence, KV head) run on one XCD, the last (most keys) first, so the K/V they all
// read stays in that XCD's L2.
//
// Block sizes 16 and 32 (a 32-token block is two 16-token sub-blocks in the pool), and 1
// (every token in its own block: the copies gather per lane, and V, token-major at that
// size, is transposed on its way into LDS).

#include <algorithm>

#include "attention_common.h"

namespace {

using namespace pkv_dev;

struct PrefillArgs {
    void* out;
    const void* q;
    const int32_t* q_start;     // [num_seqs + 1]
    const void* k_pool;
    const void* v_pool;
    const int32_t* block_tables;
    const int32_t* context_lens;
    int32_t num_seqs;
    int32_t max_blocks_per_seq;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;
    int32_t num_blocks;
    int32_t max_q_len;
    int32_t max_context_len;
    int32_t tokens_per_wg;      // TQ
    int32_t q_tiles;            // ceil(max_q_len / TQ)
    int32_t xcds;               // dies of the device: workgroup b runs on die b % xcds
    float scale_log2;
};

// Two weights as packed 16-bit heads (round to nearest even) and packed 16-bit
// remainders w - head (also rounded): one packing conversion for each pair, the heads
// widened back to float by bit operations (bf16) or a conversion (fp16).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
template <int DT>
__device__ __forceinline__ uint32_t pack2_16(float a, float b) {
    if constexpr (DT == DT_BF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
    else return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, f16x2_t));
}
template <int DT>
__device__ __forceinline__ void split_pair(float w0, float w1, int& head, int& rest) {
    const uint32_t h = pack2_16<DT>(w0, w1);
    float r0, r1;
    if constexpr (DT == DT_BF16) {
        r0 = w0 - __uint_as_float(h << 16);
        r1 = w1 - __uint_as_float(h & 0xFFFF0000u);
    } else {
        const f16x2_t hv = __builtin_bit_cast(f16x2_t, h);
        r0 = w0 - (float)hv[0];
        r1 = w1 - (float)hv[1];
    }
    head = (int)h;
    rest = (int)pack2_16<DT>(r0, r1);
}

// Rows that see at least split_keys<DT>() keys take their weights as one 16-bit rounding
// (summed into the row's denominator as rounded, so the softmax stays consistent); rows
// with fewer keys keep the 16-bit head plus remainder.  One rounding moves the output by
// sum_i w_i e_i (v_i - out), |e_i| <= u (unit roundoff: 2^-8 for bf16, 2^-11 for fp16):
// two keys of spread-out values take bf16 past the 2e-3 bar, while with scores of unit
// spread (the workloads' N(0, 1) queries and keys) the effective number of keys is
// about 0.37 x the keys seen and the error's standard deviation about
// (u / sqrt 3) / sqrt(effective keys): 1.2e-4 at 1024 bf16 keys (measured at 256 keys:
// 1.7e-3 worst over 4k-token prompts, too close to the bar), 5.8e-5 at 64 fp16 keys.
template <int DT>
constexpr int split_keys() { return DT == DT_BF16 ? 1024 : 64; }

// Four consecutive outputs (element i a multiple of 4, out 16-byte aligned) in one
// store: 16 bytes of fp32 or 8 bytes of packed 16-bit values.
template <int OUT_DT>
__device__ __forceinline__ void store_out4(void* out, int64_t i, f32x4 v) {
    if constexpr (OUT_DT == DT_F32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + i) = v;
    } else {
        const i32x2 p = {(int)pack2_16<OUT_DT>(v[0], v[1]), (int)pack2_16<OUT_DT>(v[2], v[3])};
        *reinterpret_cast<i32x2*>(static_cast<uint16_t*>(out) + i) = p;
    }
}

// ---------------------------------------------------------------------------------------
// K/V tiles staged through LDS and shared by the workgroup.
//
// The four waves of a workgroup hold different query rows of one (sequence, KV head)
// and need the same keys, so each 32-key pair of tiles is fetched once per workgroup:
// every wave copies a quarter of it from the pool straight into LDS (16-byte
// global-to-LDS loads, no registers in between), the pair after it loads while the
// current one is used, and one barrier per pair hands the buffers over.  With the K/V
// buffers out of the registers a wave fits in half the register file: two waves per
// SIMD, so one wave's exponentials and conversions run while the other's matrix
// products do.  The row sums of the weights come out of the matrix cores as well (a
// product with a block of ones), not from vector adds.
//
// Operand layout.  Every operand is one 16-byte LDS read, and the eight consecutive
// lanes that LDS serves together touch eight different 16-byte bank groups:
//  - V^T (value product, A operand): lane (dim row d, lane group q) takes the 16-byte
//    chunk of 8 consecutive tokens, tile q/2, tokens 8(q%2)..+7, of its dim.  In LDS a
//    16-dim block of a tile holds its 32 chunks (dim, half) at slot 2 dim + (half ^ bit 2
//    of dim), so dims 0..7 of one half fall in eight different slots modulo 8.
//  - The weights (B operand) must then hold those same 8 keys per lane group, so the
//    score product S^T = K . Q^T is computed with permuted key rows: in product h (of
//    two), row r stands for tile r/8, token 8((r/4)%2) + 4h + r%4.  Lane group q of the
//    output then holds, over h = 0, 1, exactly tokens 8(q%2)..+7 of tile q/2.
//  - K (score product, A operand): lane (row r, group q) reads the 16-byte chunk
//    4kk + q of its row's token; in LDS a tile's chunk c of token t sits at slot
//    16 c + (t ^ ((t & 8) >> 1)), which spreads the eight rows one LDS pass serves
//    over eight slots modulo 8.
// The copies apply these slot maps on the way in (each lane fetches the chunk that
// belongs in its slot), so the pool layout is unchanged.
//
// Column blocks of 16 query rows per wave: as many as fit two waves per SIMD in the
// registers (3 at head_dim 128: 0-3% faster than 2 at three waves per SIMD; 4 at 64;
// 2 at 256, 1.8x faster than 1).  Measured on this design with v_mfma_f32_32x32x16
// instead (one 32-query block per wave, two accumulator chains for the scores): 6-14%
// slower, although that instruction alone reaches the full matrix rate and the 16x16x32
// form about three quarters of it.
template <int D>
constexpr int lds_blocks() { return D == 64 ? 4 : D == 128 ? 3 : 2; }

template <int D, int DT, int OUT_DT, int BS, bool SPLIT>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_prefill_lds(PrefillArgs a) {
    constexpr int KI = D / 32;
    constexpr int MT = D / 16;
    constexpr int C = lds_blocks<D>();
    constexpr int RW = 16 * C;            // query rows per wave
    constexpr int TILE = BS * D;          // elements of one (block, KV head) region
    constexpr int TPB = BS >= kTile ? BS / kTile : 1;   // 16-token tiles per block
    constexpr int TE = kTile * D;         // elements of one 16-token tile
    constexpr int PIECES = TE / 512;      // 1 KiB pieces per tile: each wave copies one of each
    constexpr int STAGE = 4 * TE;         // K and V of a pair of tiles
    __shared__ __attribute__((aligned(16))) uint16_t s_kv[2 * STAGE];
    using kvec = typename std::conditional<DT == DT_BF16, bf16x8, f16x8>::type;

    // Workgroup b runs on XCD b % X (X = a.xcds, 8 on MI355X).  Pair y = sequence * KV
    // heads + KV head is given to XCD y % X (so the K/V its query tiles all read stays in
    // that XCD's L2, and with 8 KV heads on 8 dies every XCD gets one head of every
    // sequence); on each XCD the workgroups take its pairs in order, each pair's query
    // tiles last first.  The mapping is a bijection onto (pair, query tile) for any X, so
    // X only matters for speed.
    const int xcd = blockIdx.x % a.xcds, idx = blockIdx.x / a.xcds;
    const int y = xcd + a.xcds * (idx / a.q_tiles);
    if (y >= a.num_seqs * a.num_kv_heads) return;
    const int qt = a.q_tiles - 1 - idx % a.q_tiles;
    const int s = y / a.num_kv_heads;
    const int g = y - s * a.num_kv_heads;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int gq = lane & 15, quad = lane >> 4;
    const int G = a.group;

    const int32_t* trow = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
    const int r0 = sload(a.q_start, s), r1 = sload(a.q_start, s + 1);
    const int ctx = sload(a.context_lens, s);
    const int n = r1 - r0;
    if (n < 0 || n > a.max_q_len) return;          // unusable query range: rows unknown
    const int t_begin = qt * a.tokens_per_wg;
    if (t_begin >= n) return;
    const int t_end = min(n, t_begin + a.tokens_per_wg);
    const int valid_rows = (t_end - t_begin) * G;
    const bool bad_len = ctx < 1 || ctx > a.max_context_len || n > ctx;
    // Two launches share the work: SPLIT takes the workgroups whose first query sees fewer
    // than split_keys keys, the other one the rest (and writes the NaN rows of invalid
    // sequences).  The test is the same for every wave of a workgroup.
    if constexpr (SPLIT) {
        if (bad_len || ctx - n + t_begin + 1 >= split_keys<DT>()) return;
    } else {
        if (!bad_len && ctx - n + t_begin + 1 < split_keys<DT>()) return;
    }

    // this wave's rows: w*RW .. w*RW + RW - 1 of the workgroup, row = token * G + head.  A
    // wave without rows still copies its share of every tile and takes every barrier.
    const int row0 = w * RW;
    const bool has_rows = row0 < valid_rows;
    auto row_info = [&](int b, bool& live, int& tok, int& head) __attribute__((always_inline)) {
        const int r = row0 + 16 * b + gq;
        live = r < valid_rows;
        const int rr = live ? r : valid_rows - 1;       // padded rows repeat the last one
        tok = t_begin + rr / G;
        head = g * G + rr % G;
    };
    if (bad_len) {
#pragma unroll
        for (int b = 0; b < C; ++b) {
            bool live;
            int tok, head;
            row_info(b, live, tok, head);
            if (live)
                for (int e = 0; e < D / 4; ++e)
                    store_out<OUT_DT>(a.out, ((int64_t)(r0 + tok) * a.num_q_heads + head) * D +
                                                 4 * quad + 16 * (e / 4) + e % 4, NAN);
        }
        return;
    }
    int pos[C];
#pragma unroll
    for (int b = 0; b < C; ++b) {
        bool live;
        int tok, head;
        row_info(b, live, tok, head);
        pos[b] = ctx - n + tok;
    }
    // keys of the workgroup (up to its last query's position) and of this wave
    const int ntiles = (ctx - n + t_end + kTile - 1) / kTile;
    const int npairs = (ntiles + 1) / 2;
    const int last_tok = t_begin + (max(min(row0 + RW, valid_rows), 1) - 1) / G;
    const int wave_pairs = has_rows ? (ctx - n + last_tok + 2 * kTile) / (2 * kTile) : 0;
    const int pos_min = ctx - n + t_begin + row0 / G;   // this wave's first row

    kvec qop[C][KI];
#pragma unroll
    for (int b = 0; b < C; ++b) {
        bool live;
        int tok, head;
        row_info(b, live, tok, head);
        const uint16_t* qh = static_cast<const uint16_t*>(a.q) +
                             ((int64_t)(r0 + tok) * a.num_q_heads + head) * D + 8 * quad;
#pragma unroll
        for (int kk = 0; kk < KI; ++kk)
            qop[b][kk] = __builtin_bit_cast(kvec, *reinterpret_cast<const i32x4*>(qh + 32 * kk));
    }

    const uint16_t* kbase = static_cast<const uint16_t*>(a.k_pool) + (int64_t)g * TILE;
    const uint16_t* vbase = static_cast<const uint16_t*>(a.v_pool) + (int64_t)g * TILE;
    const int64_t blk_stride = (int64_t)a.num_kv_heads * TILE;
    bool bad_block = false;

    // Where pair j's tiles 2j, 2j+1 start in either pool (past the workgroup's keys: the
    // last tile again; its scores are masked and its V cleared), read a pair ahead of
    // their use.  Block sizes 16 and 32: one offset per tile, from scalar loads.  Block
    // size 1: every token has its own block, and lane l gets the offsets of token
    // kt1 = (l % 16) ^ ((l & 8) >> 1) of both tiles (vector loads of the table; tokens at
    // or past ctx take the block of token ctx - 1), which is the token whose K chunks
    // and V row the lane copies.
    const int kt1 = (lane & 15) ^ ((lane & 8) >> 1);
    auto pair_ids = [&](int j, int64_t (&off)[2]) __attribute__((always_inline)) {
        bool bad = false;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int it = min(2 * j + h, ntiles - 1);
            int32_t b;
            if constexpr (BS == 1) b = trow[min(kTile * it + kt1, ctx - 1)];
            else b = sload(trow, it / TPB);
            if ((uint32_t)b >= (uint32_t)a.num_blocks) {
                bad = true;
                b = 0;
            }
            off[h] = b * blk_stride + (BS == 1 ? 0 : (it % TPB) * TE);
        }
        if constexpr (BS == 1) bad = __ballot(bad) != 0;
        bad_block |= bad;
    };
    // Stage layout (elements): K tile 0, K tile 1 (TE each, chunks 4p..4p+3 in piece p),
    // then V as MT 1 KiB blocks [tile 0 dims 16mt..16mt+15 | tile 1 same dims], in the
    // slot orders above.  The copies are 1 KiB pieces, lane l filling slot l: K tile h
    // piece p, or V block mt (lanes 0-31 from tile 0, 32-63 from tile 1); wave w takes
    // pieces w, w + 4, ...
    constexpr int KPIECES = 2 * PIECES;
    constexpr int NPIECES = KPIECES + MT;
    static_assert(KPIECES % kWaves == 0 && MT % kWaves == 0, "pieces per wave");
    // the pool chunk that belongs in this lane's slot of a K piece / a V block
    // (both slot maps are their own inverses); block size 1: chunk lane/16 of the
    // lane's token kt1
    const int k_src = BS == 1 ? (lane >> 4) * 8 : ((lane >> 4) * 16 + kt1) * 8;
    const int v_dim = (lane & 31) >> 1;
    const int v_src = v_dim * 16 + (((lane & 1) ^ (v_dim >> 2)) & 1) * 8;
    // Block size 1 stores V token-major, so V^T chunks cannot be copied whole: lane l
    // loads 16-byte chunks (8 dims) of token kt1 of tile l / 32 into registers and
    // writes their 8 values to their slots after the pair's products.
    constexpr int CPT = D / 8;                      // 16-byte chunks of a token's V row
    constexpr int VPASS = BS == 1 ? CPT / 8 : 1;    // chunks per lane per pair
    i32x4 vrow[VPASS];
    auto issue = [&](int st, const int64_t (&off)[2]) __attribute__((always_inline)) {
        const uint16_t* k0 = kbase + off[0] + k_src;
        const uint16_t* k1 = kbase + off[1] + k_src;
        uint16_t* dst = s_kv + st * STAGE;
        if constexpr (BS == 1) {
#pragma unroll
            for (int i = 0; i < KPIECES / kWaves; ++i) {
                const int pc = w + kWaves * i;
                const int h = pc / PIECES, p = pc % PIECES;
                __builtin_amdgcn_global_load_lds((h ? k1 : k0) + p * 32, dst + h * TE + p * 512, 16, 0, 0);
            }
            const uint16_t* vr = vbase + ((lane >> 5) ? off[1] : off[0]) + ((lane >> 4) & 1) * 8;
#pragma unroll
            for (int k = 0; k < VPASS; ++k)
                vrow[k] = *reinterpret_cast<const i32x4*>(vr + 16 * (k * kWaves + w));
        } else {
            const uint16_t* vsrc = vbase + ((lane >> 5) ? off[1] : off[0]) + v_src;
#pragma unroll
            for (int i = 0; i < NPIECES / kWaves; ++i) {
                const int pc = w + kWaves * i;
                if (i < KPIECES / kWaves) {
                    const int h = pc / PIECES, p = pc % PIECES;
                    __builtin_amdgcn_global_load_lds((h ? k1 : k0) + p * 512, dst + h * TE + p * 512, 16, 0, 0);
                } else {
                    const int mt = pc - KPIECES;
                    __builtin_amdgcn_global_load_lds(vsrc + mt * 256, dst + 2 * TE + mt * 512, 16, 0, 0);
                }
            }
        }
    };
    // block size 1: chunk c = 2 (k * 4 + w) + (l / 16) % 2 of the lane's V row (dims
    // 8c .. 8c+7, all in block mt = c / 2) into slot 2 d + (half ^ bit 2 of d), element
    // kt1 % 8, of tile l / 32 (d = dim % 16, half = kt1 / 8)
    auto store_v = [&](int st) __attribute__((always_inline)) {
        if constexpr (BS == 1) {
            const int half = kt1 >> 3;
            uint16_t* vb = s_kv + st * STAGE + 2 * TE + (lane >> 5) * 256 + ((lane >> 4) & 1) * 128 + (kt1 & 7);
#pragma unroll
            for (int k = 0; k < VPASS; ++k) {
                uint16_t* vk = vb + (k * kWaves + w) * 512;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t x = (uint32_t)vrow[k][e >> 1];
                    vk[(2 * e + (half ^ (e >> 2))) * 8] = (uint16_t)(e & 1 ? x >> 16 : x);
                }
            }
        }
    };

    f32x4 acc[C][MT], accl[C];
    float m[C];
#pragma unroll
    for (int b = 0; b < C; ++b) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[b][mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
        accl[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
        m[b] = kNegInf;
    }
    // A-operand of ones: the product with the weights gives each row's weight sum
    const int one2 = DT == DT_BF16 ? 0x3F803F80 : 0x3C003C00;
    const i32x4 ones = {one2, one2, one2, one2};

    auto mfma = [&](const i32x4& x, const i32x4& yv, f32x4 c) __attribute__((always_inline)) {
        if constexpr (DT == DT_BF16)
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x),
                                                          __builtin_bit_cast(bf16x8, yv), c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, x),
                                                         __builtin_bit_cast(f16x8, yv), c, 0, 0, 0);
    };

    // per-lane LDS read offsets within a stage: K rows of score product h (tile gq/8,
    // token 8((gq/4)%2) + 4h + gq%4, chunk 4kk + quad) and the V^T chunk
    int k_rd[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int t = 8 * ((gq >> 2) & 1) + 4 * h + (gq & 3);
        k_rd[h] = (gq >> 3) * TE + (quad * 16 + (t ^ ((t & 8) >> 1))) * 8;
    }
    const int v_rd = 2 * TE + (quad >> 1) * 256 + (2 * gq + (((quad & 1) ^ (gq >> 2)) & 1)) * 8;

    // one pair of tiles from LDS stage `stg`
    auto compute = [&](auto special, int j, const uint16_t* stg) __attribute__((always_inline)) {
        // The score products run at raised priority: the SIMD's other wave, in its
        // softmax, then fills the gaps between them (measured 1-2% faster; raising the
        // value products' priority as well measured slower). Not at block size 1, where it
        // measured 9% slower (that path's per-lane table reads and V stores sit between
        // the products).
        if constexpr (BS != 1) __builtin_amdgcn_s_setprio(1);
        f32x4 sc[C][2];
#pragma unroll
        for (int b = 0; b < C; ++b) sc[b][0] = sc[b][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int kk = 0; kk < KI; ++kk) {
                const i32x4 kop = *reinterpret_cast<const i32x4*>(stg + k_rd[h] + kk * 512);
#pragma unroll
                for (int b = 0; b < C; ++b)
                    sc[b][h] = mfma(kop, __builtin_bit_cast(i32x4, qop[b][kk]), sc[b][h]);
            }
        }
        if constexpr (BS != 1) __builtin_amdgcn_s_setprio(0);
        if (decltype(special)::value && (2 * j + 1) * kTile + kTile - 1 > pos_min) {
            // lane group q holds tile q/2, tokens 8(q%2) + 4h + r
            const int kp0 = (2 * j + (quad >> 1)) * kTile + 8 * (quad & 1);
#pragma unroll
            for (int b = 0; b < C; ++b)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (kp0 + 4 * h + r > pos[b]) sc[b][h][r] = kNegInf;
        }
        float xm[C];
        bool grow = false;
#pragma unroll
        for (int b = 0; b < C; ++b) {
            float t = fmaxf(fmaxf(sc[b][0][0], sc[b][0][1]), sc[b][0][2]);
            t = fmaxf(fmaxf(t, sc[b][0][3]), sc[b][1][0]);
            t = fmaxf(fmaxf(t, sc[b][1][1]), sc[b][1][2]);
            t = fmaxf(t, sc[b][1][3]);
            xm[b] = t * a.scale_log2;
            grow |= xm[b] > m[b] + kRescaleSlack;
        }
        if (__ballot(grow)) {
#pragma unroll
            for (int b = 0; b < C; ++b) {
                const float mnew = fmaxf(m[b], max_across_quads(xm[b]));
                const float alpha = exp2_fast(m[b] - mnew);
                accl[b] *= alpha;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[b][mt] *= alpha;
                m[b] = mnew;
            }
        }
        // Block by block at head_dim 128 with blocks of 16/32 tokens: a block's weights,
        // their row sums and its value products, so that its matrix products run while
        // the next block's exponentials are computed, the V^T operands held for the whole
        // pair (whole prompts 0.379 -> 0.384 of peak, three alternating runs; head_dim 64
        // measured slower, and 256 and block size 1 lack the registers).  Otherwise all
        // weights first, then the value products operand by operand.  Same products in
        // the same order either way.
        if constexpr (D == 128 && BS != 1) {
            // V^T operands of the pair (tile q/2, tokens 8(q%2)..+7 of dim 16 mt + gq),
            // read once for all blocks; slots past the context may hold anything, NaN
            // included: cleared
            const int vt = 2 * j + (quad >> 1);
            const int vvalid = (vt < ntiles ? ctx - vt * kTile : 0) - 8 * (quad & 1);
            i32x4 va[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                va[mt] = *reinterpret_cast<const i32x4*>(stg + v_rd + mt * 512);
                if (decltype(special)::value && vvalid < 8) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        uint32_t x = (uint32_t)va[mt][e];
                        if (2 * e >= vvalid) x &= 0xFFFF0000u;
                        if (2 * e + 1 >= vvalid) x &= 0x0000FFFFu;
                        va[mt][e] = (int)x;
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < C; ++b) {
                i32x4 phi, plo;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p0 = exp2_fast(fmaf(sc[b][r >> 1][2 * (r & 1)], a.scale_log2, -m[b]));
                    const float p1 = exp2_fast(fmaf(sc[b][r >> 1][2 * (r & 1) + 1], a.scale_log2, -m[b]));
                    if constexpr (SPLIT) {
                        int hw, lw;
                        split_pair<DT>(p0, p1, hw, lw);
                        phi[r] = hw;
                        plo[r] = lw;
                    } else {
                        phi[r] = (int)pack2_16<DT>(p0, p1);
                    }
                }
                accl[b] = mfma(ones, phi, accl[b]);
                if constexpr (SPLIT) accl[b] = mfma(ones, plo, accl[b]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    acc[b][mt] = mfma(va[mt], phi, acc[b][mt]);
                    if constexpr (SPLIT) acc[b][mt] = mfma(va[mt], plo, acc[b][mt]);
                }
            }
        } else {
            i32x4 phi[C], plo[C];
#pragma unroll
            for (int b = 0; b < C; ++b) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p0 = exp2_fast(fmaf(sc[b][r >> 1][2 * (r & 1)], a.scale_log2, -m[b]));
                    const float p1 = exp2_fast(fmaf(sc[b][r >> 1][2 * (r & 1) + 1], a.scale_log2, -m[b]));
                    if constexpr (SPLIT) {
                        int hw, lw;
                        split_pair<DT>(p0, p1, hw, lw);
                        phi[b][r] = hw;
                        plo[b][r] = lw;
                    } else {
                        phi[b][r] = (int)pack2_16<DT>(p0, p1);
                    }
                }
                accl[b] = mfma(ones, phi[b], accl[b]);
                if constexpr (SPLIT) accl[b] = mfma(ones, plo[b], accl[b]);
            }
            // V^T operand: tile q/2, tokens 8(q%2)..+7 of dim 16 mt + gq (slots past the
            // context may hold anything, NaN included: cleared)
            const int vt = 2 * j + (quad >> 1);
            const int vvalid = (vt < ntiles ? ctx - vt * kTile : 0) - 8 * (quad & 1);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                i32x4 va = *reinterpret_cast<const i32x4*>(stg + v_rd + mt * 512);
                if (decltype(special)::value && vvalid < 8) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        uint32_t x = (uint32_t)va[e];
                        if (2 * e >= vvalid) x &= 0xFFFF0000u;
                        if (2 * e + 1 >= vvalid) x &= 0x0000FFFFu;
                        va[e] = (int)x;
                    }
                }
#pragma unroll
                for (int b = 0; b < C; ++b) {
                    acc[b][mt] = mfma(va, phi[b], acc[b][mt]);
                    if constexpr (SPLIT) acc[b][mt] = mfma(va, plo[b], acc[b][mt]);
                }
            }
        }
    };

    constexpr std::integral_constant<bool, false> kPlain{};
    constexpr std::integral_constant<bool, true> kSpecial{};
    // pairs before j_plain need neither the causal mask nor V clearing for this wave
    const int t_zero = min(ntiles, ctx / kTile);
    const int j_mask = (pos_min + 1) / (2 * kTile);
    const int j_plain = min(min(j_mask, t_zero / 2), wave_pairs);

    // Pair j sits in stage j & 1.  At the barrier of step j every wave has finished pair
    // j - 1 (so its stage may be overwritten by pair j + 1) and every copy of pair j has
    // landed (each wave waits for its own copies before the barrier).
    int64_t ids_next[2], ids_after[2];
    pair_ids(0, ids_next);
    issue(0, ids_next);
    store_v(0);
    pair_ids(min(1, npairs - 1), ids_next);
    int j = 0;
    for (; j < j_plain; ++j) {
        wait_memory_done();
        __syncthreads();
        if (j + 1 < npairs) issue((j + 1) & 1, ids_next);
        pair_ids(min(j + 2, npairs - 1), ids_after);
        compute(kPlain, j, s_kv + (j & 1) * STAGE);
        if (j + 1 < npairs) store_v((j + 1) & 1);
        ids_next[0] = ids_after[0];
        ids_next[1] = ids_after[1];
    }
    for (; j < npairs; ++j) {
        wait_memory_done();
        __syncthreads();
        if (j + 1 < npairs) issue((j + 1) & 1, ids_next);
        pair_ids(min(j + 2, npairs - 1), ids_after);
        if (j < wave_pairs) compute(kSpecial, j, s_kv + (j & 1) * STAGE);
        if (j + 1 < npairs) store_v((j + 1) & 1);
        ids_next[0] = ids_after[0];
        ids_next[1] = ids_after[1];
    }
    if (!has_rows) return;

    // normalise and write: lane holds row gq of block b, dims 16*mt + 4*quad .. +3
#pragma unroll
    for (int b = 0; b < C; ++b) {
        const float inv = 1.f / accl[b][0];
        bool live;
        int tok, head;
        row_info(b, live, tok, head);
        if (!live) continue;
        const int64_t ob = ((int64_t)(r0 + tok) * a.num_q_heads + head) * D;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            f32x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = bad_block ? NAN : acc[b][mt][r] * inv;
            store_out4<OUT_DT>(a.out, ob + 16 * mt + 4 * quad, v);
        }
    }
}

// Two launches: every query tile without the weight split, then (only the first tiles of
// each sequence can hold queries that see fewer than split_keys keys) those tiles with it.
template <int D, int DT, int OUT, int BS>
void launch_t(const PrefillArgs& a, dim3 grid, hipStream_t st) {
    PrefillArgs b = a;
    b.q_tiles = std::min(a.q_tiles, (split_keys<DT>() - 1 + a.tokens_per_wg - 1) / a.tokens_per_wg);
    const int64_t pairs = (int64_t)a.num_seqs * a.num_kv_heads;
    const dim3 g2((unsigned)((int64_t)a.xcds * b.q_tiles * ((pairs + a.xcds - 1) / a.xcds)));
    attn_prefill_lds<D, DT, OUT, BS, false><<<grid, dim3(kWaves * 64), 0, st>>>(a);
    attn_prefill_lds<D, DT, OUT, BS, true><<<g2, dim3(kWaves * 64), 0, st>>>(b);
}

template <int D, int DT, int BS>
void launch_o(const PrefillArgs& a, int out_dtype, dim3 grid, hipStream_t st) {
    if (out_dtype == PAGED_KV_F32) launch_t<D, DT, DT_F32, BS>(a, grid, st);
    else launch_t<D, DT, DT, BS>(a, grid, st);
}

template <int D, int BS>
void launch_dt(const PrefillArgs& a, int dtype, int out_dtype, dim3 grid, hipStream_t st) {
    if (dtype == PAGED_KV_F16) launch_o<D, DT_F16, BS>(a, out_dtype, grid, st);
    else launch_o<D, DT_BF16, BS>(a, out_dtype, grid, st);
}

template <int D>
void launch_bs(const PrefillArgs& a, int bs, int dtype, int out_dtype, dim3 grid, hipStream_t st) {
    if (bs == 32) launch_dt<D, 32>(a, dtype, out_dtype, grid, st);
    else if (bs == 1) launch_dt<D, 1>(a, dtype, out_dtype, grid, st);
    else launch_dt<D, 16>(a, dtype, out_dtype, grid, st);
}

// query tokens per workgroup: its 4 waves' rows (16 per column block) over the group
int tokens_per_workgroup(int head_dim, int group) {
    const int blocks = head_dim == 64 ? lds_blocks<64>() : head_dim == 256 ? lds_blocks<256>() : lds_blocks<128>();
    return 4 * 16 * blocks / group;
}

paged_kv_status launch_status(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        pkv::set_error("%s launch failed: %s", what, hipGetErrorString(e));
        return PAGED_KV_ERR_HIP;
    }
    return PAGED_KV_OK;
}

}  // namespace

extern "C" {

paged_kv_status paged_attention_prefill(const paged_kv_pool_desc* desc, void* out,
                                        int32_t out_dtype, const void* q, const int32_t* q_start,
                                        const void* k_pool, const void* v_pool,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t max_q_len,
                                        int32_t max_context_len, float scale, void* stream) {
    pkv::clear_error();
    if (!pkv::kernel_desc(desc, true)) return PAGED_KV_ERR_INVALID_ARG;
    if (desc->dtype == PAGED_KV_F32) {
        pkv::set_error("prefill attention needs fp16/bf16 pools");
        return PAGED_KV_ERR_UNSUPPORTED;
    }
    if (num_seqs < 0 || num_q_heads < 1 || num_q_heads % desc->num_kv_heads) {
        pkv::set_error("num_seqs %d < 0, or num_q_heads %d not a positive multiple of %d",
                       num_seqs, num_q_heads, desc->num_kv_heads);
        return PAGED_KV_ERR_INVALID_ARG;
    }
    const int group = num_q_heads / desc->num_kv_heads;
    if (group > 16) {
        pkv::set_error("at most 16 query heads per KV head (got %d)", group);
        return PAGED_KV_ERR_UNSUPPORTED;
    }
    if (out_dtype != desc->dtype && out_dtype != PAGED_KV_F32) {
        pkv::set_error("out_dtype must be the pool dtype or fp32");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    if (!(scale > 0.f)) {
        pkv::set_error("prefill attention needs scale > 0 (got %g)", (double)scale);
        return PAGED_KV_ERR_INVALID_ARG;
    }
    if (max_context_len < 1 || max_q_len < 0 || max_q_len > max_context_len) {
        pkv::set_error("need 0 <= max_q_len (%d) <= max_context_len (%d), max_context_len >= 1",
                       max_q_len, max_context_len);
        return PAGED_KV_ERR_INVALID_ARG;
    }
    if ((int64_t)max_blocks_per_seq * desc->block_size < max_context_len) {
        pkv::set_error("max_blocks_per_seq %d cannot hold max_context_len %d", max_blocks_per_seq,
                       max_context_len);
        return PAGED_KV_ERR_INVALID_ARG;
    }
    if (num_seqs == 0 || max_q_len == 0) return PAGED_KV_OK;
    if (!out || !q || !q_start || !k_pool || !v_pool || !block_tables || !context_lens) {
        pkv::set_error("null pointer argument");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    if ((reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(q) |
         reinterpret_cast<uintptr_t>(k_pool) | reinterpret_cast<uintptr_t>(v_pool)) & 15) {
        pkv::set_error("out, q and pools must be 16-byte aligned");
        return PAGED_KV_ERR_INVALID_ARG;
    }
    PrefillArgs a;
    a.out = out;
    a.q = q;
    a.q_start = q_start;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.num_seqs = num_seqs;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = desc->num_kv_heads;
    a.group = group;
    a.num_blocks = desc->num_blocks;
    a.max_q_len = max_q_len;
    a.max_context_len = max_context_len;
    a.tokens_per_wg = tokens_per_workgroup(desc->head_dim, group);
    a.q_tiles = (max_q_len + a.tokens_per_wg - 1) / a.tokens_per_wg;
    a.scale_log2 = scale * kLog2e;
    a.xcds = pkv::device_shape().xcds;
    const int64_t pairs = (int64_t)num_seqs * desc->num_kv_heads;
    const int64_t wgs = (int64_t)a.xcds * a.q_tiles * ((pairs + a.xcds - 1) / a.xcds);
    if (wgs > INT32_MAX) {
        pkv::set_error("too many (sequence, KV head, query tile) workgroups for one launch");
        return PAGED_KV_ERR_UNSUPPORTED;
    }
    const dim3 grid((unsigned)wgs);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    switch (desc->head_dim) {
        case 64: launch_bs<64>(a, desc->block_size, desc->dtype, out_dtype, grid, st); break;
        case 256: launch_bs<256>(a, desc->block_size, desc->dtype, out_dtype, grid, st); break;
        default: launch_bs<128>(a, desc->block_size, desc->dtype, out_dtype, grid, st); break;
    }
    return launch_status("paged attention prefill kernel");
}

}  // extern "C"
