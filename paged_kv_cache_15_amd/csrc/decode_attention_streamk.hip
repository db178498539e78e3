// Stream-K paged decode attention for gfx950.
//
// Same computation as the fixed-partition kernels (deepsonar "PagedAttention de vLLM
// …" §2.2/§2.6: gather a sequence's blocks through its table; deeplearn.tn
// "PagedAttention : comment optimiser la mémoire GPU …", PagedAttention vs.
// FlashAttention: stream K/V tiles through on-chip memory with an incremental
// softmax), scheduled differently:
//
// Every (sequence, head unit, 16-token tile) of the batch is a tile; tiles are laid on
// one line ordered by sequence, then unit, then position.  A fixed number W of waves
// each take a contiguous slice of the line (equal to within one tile, or weighted by
// the XCD the wave runs on: see SliceMap) and stream it with a two-deep load pipeline
// that never restarts at sequence or head boundaries.  When a
// wave's slice covers a whole (sequence, unit) the wave writes the normalised output;
// otherwise it writes the piece's (max, sum, weighted values), counts it in a per-unit
// counter, and the wave that completes the count merges the unit's pieces in slice
// order (log-sum-exp) — no second kernel.  Piece index = wave index + (sequence, unit)
// index: along the line every wave boundary and every unit boundary starts a new piece,
// so this numbering is dense and collision-free.
//
// Units: the MFMA kernel's unit is a KV head with its group of query heads (fp16/bf16,
// group >= 2); the VALU kernel's unit is one query head.
//
// Block sizes: with 16 or 32 tokens per block a tile is one block or one of its two
// 16-token sub-blocks (stored one after the other, each laid out like a 16-token block);
// with 1 token per block a tile gathers 16 blocks (per-lane addresses, and V transposed
// through LDS, since such a pool stores each token's values as one row).
//
// Results depend only on the logical token order, W and the slice weights, never on
// where blocks sit in the pool: placement and sharing leave them bit-identical.

#include "attention_common.h"
#include "attention_host.h"

namespace {

using namespace pkv_dev;

struct StreamArgs {
    void* out;
    const void* q;
    const void* k_pool;
    const void* v_pool;
    const int32_t* block_tables;
    const int32_t* context_lens;
    int32_t* counters; // per unit: pieces written so far; zero on entry, left zero
    float* ws_m;
    float* ws_l;
    float* ws_acc;
    int32_t num_seqs;
    int32_t max_blocks_per_seq;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;           // query heads per KV head
    int32_t units;           // head units per sequence
    int32_t heads_per_unit;  // query heads per unit
    int32_t num_blocks;
    int32_t max_context_len;
    int32_t waves;           // W
    int32_t weight_odd;      // slice weight of a wave of an odd workgroup (even: kWeightEven)
    float scale_log2;
    // partition states (attn_mfma_streamk<..., true>): see pkv::StreamLaunch
    int32_t pm_tiles;
    int32_t pm_max_parts;
    float* pm_m;
    float* pm_l;
    float* pm_acc;
};

__device__ __forceinline__ int tiles_of(int ctx, int max_ctx) {
    return (ctx >= 1 && ctx <= max_ctx) ? (ctx + kTile - 1) / kTile : 0;
}

// Exclusive prefix of per-sequence tile counts (per unit) into s_pref[0..B]; returns
// s_pref[B].  Called by every thread of the workgroup.
__device__ int build_prefix(const StreamArgs& a, int* s_pref) {
    __shared__ int s_wsum[kWaves];
    const int B = a.num_seqs, tid = threadIdx.x, nthr = blockDim.x;
    const int lane = tid & 63, w = tid >> 6;
    // tile counts into LDS with coalesced loads, several in flight per thread
#pragma unroll 8
    for (int i = tid; i < B; i += nthr) s_pref[i] = tiles_of(a.context_lens[i], a.max_context_len);
    __syncthreads();
    const int chunk = (B + nthr - 1) / nthr;
    const int lo = min(B, tid * chunk), hi = min(B, lo + chunk);
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += s_pref[i];
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
    }
    if (lane == 63) s_wsum[w] = incl;
    __syncthreads();
    int off = 0;
    for (int ww = 0; ww < w; ++ww) off += s_wsum[ww];
    int run = off + incl - sum;
    for (int i = lo; i < hi; ++i) {
        const int v = s_pref[i];
        s_pref[i] = run;
        run += v;
    }
    if (tid == nthr - 1) s_pref[B] = off + incl;
    __syncthreads();
    return s_pref[B];
}

// Position on the tile line, kept in scalar registers (every value is wave-uniform).
struct Cursor {
    int s, u, it, nt, ctx;
};

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Cursor of tile t: sequence = the last s with units * pref[s] <= t (it has >= 1 tile).
__device__ Cursor locate(const StreamArgs& a, const int* s_pref, int64_t t) {
    int lo = 0, hi = a.num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)a.units * uni(s_pref[mid]) <= t) lo = mid;
        else hi = mid - 1;
    }
    Cursor c;
    c.s = lo;
    const int base = uni(s_pref[lo]);
    c.nt = uni(s_pref[lo + 1]) - base;
    const int64_t o = t - (int64_t)a.units * base;
    c.u = (int)(o / c.nt);
    c.it = (int)(o - (int64_t)c.u * c.nt);
    c.ctx = sload(a.context_lens, lo);
    return c;
}

// Next tile on the line (only called while one exists).
__device__ __forceinline__ void advance(const StreamArgs& a, Cursor& c) {
    if (++c.it < c.nt) return;
    c.it = 0;
    if (++c.u < a.units) return;
    c.u = 0;
    do {
        ++c.s;
        c.ctx = sload(a.context_lens, c.s);
        c.nt = tiles_of(c.ctx, a.max_context_len);
    } while (c.nt == 0 && c.s < a.num_seqs - 1);
}

// Physical block of the cursor's tile (block size BS >= 16: the tile is sub-block
// it % TPB of block it / TPB); out-of-range ids read block 0 and flag the unit.
template <int BS>
__device__ __forceinline__ int32_t tile_block(const StreamArgs& a, const Cursor& c, bool& bad) {
    const int32_t bid = sload(a.block_tables, (int64_t)c.s * a.max_blocks_per_seq + c.it / (BS / kTile));
    bad = (uint32_t)bid >= (uint32_t)a.num_blocks;
    return bad ? 0 : bid;
}

// Slices may be weighted by the XCD their wave runs on.  Workgroup b is dispatched to
// XCD b % 8, and on MI355X the odd XCDs stream the one-wave-per-SIMD launches (head_dim
// 128 and up, 16- or 32-token blocks) about 10% slower than the even ones (measured
// per-wave rates on the GQA workload: 0.77 against 0.855 tiles/us, the only systematic
// spread left), so a wave of an odd workgroup gets w_odd / kWeightEven of an even
// wave's share (w_odd = StreamArgs::weight_odd; equal weights elsewhere, where the
// weighting measured slower).  Wave j belongs to workgroup j / kWaves; S(j), the weight
// of waves 0 .. j-1, has a closed form, and so has its inverse, which the merge needs
// to find the waves that hold a unit's pieces.
constexpr int64_t kWeightEven = 64;

struct SliceMap {
    int64_t T;     // tiles on the line
    int W;         // waves
    int64_t wo;    // weight of an odd workgroup's wave
    __device__ int64_t pair_weight() const { return kWaves * (kWeightEven + wo); }
    __device__ int64_t weight_before(int64_t j) const {
        const int64_t p = j / (2 * kWaves), r = j - p * 2 * kWaves;
        return p * pair_weight() + (r < kWaves ? r * kWeightEven
                                               : kWaves * kWeightEven + (r - kWaves) * wo);
    }
    // first tile of wave j's slice: floor(T S(j) / S(W))
    __device__ int64_t start(int64_t j) const { return T * weight_before(j) / weight_before(W); }
    // the wave whose slice holds tile t: the largest j with floor(T S(j) / S(W)) <= t,
    // i.e. with S(j) <= M = floor(((t + 1) S(W) - 1) / T)
    __device__ int wave_of(int64_t t) const {
        const int64_t M = ((t + 1) * weight_before(W) - 1) / T;
        const int64_t p = M / pair_weight(), rem = M - p * pair_weight();
        const int64_t r = rem < kWaves * kWeightEven ? rem / kWeightEven
                                                     : kWaves + (rem - kWaves * kWeightEven) / wo;
        return (int)min(p * 2 * kWaves + r, (int64_t)W - 1);
    }
    // with few tiles per wave some slices are empty; those waves wrote no piece
    __device__ bool empty(int j) const { return start(j + 1) == start(j); }
    // no slice is empty when the lightest wave's share is at least one tile
    __device__ bool dense() const { return T * min(wo, kWeightEven) >= weight_before(W); }
};

__device__ __forceinline__ SliceMap slice_map(const StreamArgs& a, int64_t T) {
    return SliceMap{T, a.waves, (int64_t)a.weight_odd};
}

__device__ __forceinline__ void wave_slice(const StreamArgs& a, int64_t T, int j, int64_t& t0,
                                           int64_t& t1) {
    const SliceMap sm = slice_map(a, T);
    t0 = sm.start(j);
    t1 = sm.start(j + 1);
}

// Number of pieces unit q was cut into (its tiles start at line position ta).
__device__ __forceinline__ int unit_pieces(const SliceMap& sm, int64_t ta, int nt, int& jf, int& jl) {
    jf = sm.wave_of(ta);
    jl = sm.wave_of(ta + nt - 1);
    if (sm.dense()) return jl - jf + 1;
    int cnt = 0;
    for (int jj = jf; jj <= jl; ++jj) cnt += !sm.empty(jj);
    return cnt;
}

// Pieces cross XCDs, whose L2 caches are not kept coherent with each other inside a
// kernel: they are written and read with put_coherent / get_coherent (see
// attention_common.h), so publishing a piece only needs its stores to have completed
// before the counter is bumped.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kPolicySc1 = 1 << 4;   // cache-policy operand bit of sc1 on gfx94x/gfx950
// 16-byte form of put_coherent for a wave-uniform region of `bytes` bytes at `base`
// (a buffer store with the same sc1 policy); lanes whose offset falls outside the
// region write nothing (the buffer's range check drops them).
__device__ __forceinline__ void put_coherent4(float* base, uint32_t bytes, uint32_t off_bytes,
                                              f32x4 v) {
    // third descriptor word 0x00020000: raw 32-bit data format on gfx9-family chips
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off_bytes, 0,
                                           kPolicySc1);
}

// Log-sum-exp merge of all pieces of unit q (written by waves jf..jl; empty slices wrote
// none), in slice order, into the unit's G query-head output rows.  One wave, heads in
// groups of HC: lane h < HC keeps head g0+h's running max M and sum L, and every lane
// holds the group's output elements idx = lane + 64 i (head 64 i / D, uniform).
// Pieces are folded in online, PC at a time, all loads of a chunk in flight together:
//   M' = max(M, m_p), L' = L 2^(M - M') + l_p 2^(m_p - M'), acc likewise; out = acc / L.
// The code is kept small on purpose: every wave reaches it at the end of the launch
// with a cold instruction cache.
template <int D, int OUT_DT, int HC, int PC>
__device__ void merge_unit(const StreamArgs& a, int q, int s, int u, int jf, int jl, int64_t T,
                           int lane) {
    constexpr int EC = HC * D / 64;       // outputs per lane per head group
    const int G = a.heads_per_unit;
    const SliceMap sm = slice_map(a, T);
    const bool dense = sm.dense();
#pragma unroll 1
    for (int g0 = 0; g0 < G; g0 += HC) {
        float Ml = kNegInf, Ll = 0.f, acc[EC];
#pragma unroll
        for (int i = 0; i < EC; ++i) acc[i] = 0.f;
        bool bad = false;
        const int hl = min(g0 + min(lane, HC - 1), G - 1);
#pragma unroll 1
        for (int k0 = jf; k0 <= jl; k0 += PC) {
            // Loads first, with no branch between them: slots past jl re-read piece jl
            // and padded heads re-read head G-1; neither is folded in.
            float pm[PC], pl[PC], pa[PC][EC];
#pragma unroll
            for (int p = 0; p < PC; ++p) {
                const int64_t pr = ((int64_t)min(k0 + p, jl) + q) * G;
                pm[p] = get_coherent(a.ws_m + pr + hl);
                pl[p] = get_coherent(a.ws_l + pr + hl);
#pragma unroll
                for (int i = 0; i < EC; ++i) {
                    const int hi = min(g0 + 64 * i / D, G - 1);
                    pa[p][i] = get_coherent(a.ws_acc + (pr + hi) * D + (64 * i) % D + lane);
                }
            }
#pragma unroll
            for (int p = 0; p < PC; ++p) {
                const int jj = k0 + p;
                if (jj > jl || (!dense && sm.empty(jj))) continue;
                bad |= __ballot(pm[p] != pm[p]) != 0;
                const float mn = fmaxf(Ml, pm[p]);
                const float sc = exp2_fast(Ml - mn), wt = exp2_fast(pm[p] - mn);
                Ll = Ll * sc + wt * pl[p];
                Ml = mn;
#pragma unroll
                for (int i = 0; i < EC; ++i) {
                    const int h = 64 * i / D;
                    const float sh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), h));
                    const float wh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), h));
                    acc[i] = acc[i] * sh + wh * pa[p][i];
                }
            }
        }
        const int64_t ob = ((int64_t)s * a.num_q_heads + u * G + g0) * D + lane;
        const float inv = 1.f / Ll;
#pragma unroll
        for (int i = 0; i < EC; ++i) {
            const int h = 64 * i / D;
            const float ih = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inv), h));
            if (g0 + h < G) store_out<OUT_DT>(a.out, ob + 64 * i, bad ? NAN : acc[i] * ih);
        }
    }
}

// Units this wave wrote a piece of (at most two: the first unit of its slice, if it
// began in an earlier slice, and the last, if it goes on into a later one).
struct Pending {
    int n = 0;
    int s0 = 0, u0 = 0, nt0 = 0, s1 = 0, u1 = 0, nt1 = 0;
    __device__ void add(int s, int u, int nt) {
        if (n == 0) { s0 = s; u0 = u; nt0 = nt; }
        else { s1 = s; u1 = u; nt1 = nt; }
        ++n;
    }
};

// End of a wave's slice: once its pieces (written with put_coherent) have completed, it
// counts them in their units' counters; for each unit it counted last, it merges the
// pieces (reading with get_coherent, after the count came back) and resets the
// counter for the next call.  Counting only here keeps the wait for the piece stores
// out of the load pipeline.
template <int D, int OUT_DT, int HC, int PC>
__device__ void publish_pieces(const StreamArgs& a, const int* s_pref, const Pending& pd,
                               int64_t T, int lane) {
    if (pd.n == 0) return;
    wait_memory_done();
    const int q0 = pd.s0 * a.units + pd.u0, q1 = pd.s1 * a.units + pd.u1;
    int old0 = 0, old1 = 0;
    if (lane == 0) {
        old0 = __hip_atomic_fetch_add(a.counters + q0, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (pd.n > 1)
            old1 = __hip_atomic_fetch_add(a.counters + q1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    old0 = __shfl(old0, 0);
    old1 = __shfl(old1, 0);
    // Ordering of the merge's reads after the count, stated for gfx950: every piece was
    // stored with the sc1 policy (written through to the device-coherent level, not kept
    // dirty in the XCD's own L2), and its writer bumped the counter only after
    // s_waitcnt vmcnt(0) had seen those stores acknowledged.  The counter is an
    // agent-scope atomic, performed at that coherent level, so a bump that returns the
    // final count comes after every other writer's pieces are there, and the merge reads
    // them with sc1 loads, which do not hit stale lines in this XCD's L2.  What the
    // hardware does not order for us is the compiler: this fence keeps it from moving
    // the merge's loads above the counter's atomic (an agent-scope acquire fence would
    // also invalidate the L2 here, which the sc1 loads already make unnecessary).
    __atomic_signal_fence(__ATOMIC_ACQUIRE);
#pragma unroll 1
    for (int e = 0; e < pd.n; ++e) {
        const int s = e ? pd.s1 : pd.s0, u = e ? pd.u1 : pd.u0, nt = e ? pd.nt1 : pd.nt0;
        const int q = e ? q1 : q0, old = e ? old1 : old0;
        int jf, jl;
        const int64_t ta = (int64_t)a.units * uni(s_pref[s]) + (int64_t)u * nt;
        if (old != unit_pieces(slice_map(a, T), ta, nt, jf, jl) - 1) continue;
        merge_unit<D, OUT_DT, HC, PC>(a, q, s, u, jf, jl, T, lane);
        if (lane == 0) __hip_atomic_store(a.counters + q, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Sequences with an invalid length (no tiles: s_pref[s + 1] == s_pref[s]) get NaN
// outputs; workgroup b takes sequences b, b + grid, ...  Only LDS is read, so no
// workgroup's own slice is held up by this.
template <int D, int OUT_DT>
__device__ void nan_invalid_sequences(const StreamArgs& a, const int* s_pref) {
    for (int s = blockIdx.x; s < a.num_seqs; s += gridDim.x) {
        if (s_pref[s + 1] != s_pref[s]) continue;
        const int64_t ob = (int64_t)s * a.num_q_heads * D;
        for (int i = threadIdx.x; i < a.num_q_heads * D; i += blockDim.x)
            store_out<OUT_DT>(a.out, ob + i, NAN);
    }
}

// ---------------------------------------------------------------------------------
// MFMA stream-K kernel (fp16/bf16, 2..16 query heads per KV head).  The per-tile math
// is the fixed-partition MFMA kernel's: S^T = K.Q^T with 16x16x32 MFMAs, lazy-rescaled
// base-2 softmax, O^T += V^T.P^T with P split into 16-bit head + remainder.
// ---------------------------------------------------------------------------------
// Floats of LDS per wave that hold finished partition pieces (PM): 30 KiB (block size 1,
// whose tiles also pass through LDS: 8 KiB).
template <int BS>
constexpr int kPmWaveFloats() { return BS == 1 ? 2048 : 7680; }

// PM: partition states instead of outputs (pkv::StreamLaunch::pm_tiles).  Slices are then
// at least two partitions long (fewer waves take part when the batch is small), so a
// partition is cut at most once: into the piece that holds its first tile and the rest.
template <int D, int DT, int OUT_DT, int BS, bool PM>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(mfma_waves_per_simd<D, true>())))
void attn_mfma_streamk(StreamArgs a) {
    constexpr int KI = D / 32;
    constexpr int MT = D / 16;
    constexpr int TILE = BS * D;          // elements of one (block, KV head) region
    constexpr int TPB = BS >= kTile ? BS / kTile : 1;   // tiles per block
    constexpr int LDW = D + 8;            // block size 1: LDS row of one token's values
    using kvec = typename std::conditional<DT == DT_BF16, bf16x8, f16x8>::type;
    // V registers as loaded: a V^T operand per 16 dims, or (block size 1) token rows
    using vbuf = typename std::conditional<BS == 1, i32x4[KI], i32x2[MT]>::type;
    __shared__ uint16_t s_vt[BS == 1 ? kWaves * kTile * LDW : 1];
    __shared__ uint16_t s_kt[BS == 1 ? kWaves * kTile * LDW : 1];
    __shared__ __attribute__((aligned(16))) float s_pm[PM ? kWaves * kPmWaveFloats<BS>() : 4];

    extern __shared__ int s_pref[];
    const int tiles_per_unit = build_prefix(a, s_pref);
    nan_invalid_sequences<D, OUT_DT>(a, s_pref);
    const int lane = threadIdx.x & 63;
    const int j = uni(blockIdx.x * kWaves + (threadIdx.x >> 6));
    if (j >= a.waves) return;
    const int64_t T = (int64_t)a.units * tiles_per_unit;
    int64_t t0, t1;
    if constexpr (PM) {
        const int W = (int)max<int64_t>(1, min<int64_t>(a.waves, T / (2 * a.pm_tiles)));
        if (j >= W) return;
        const SliceMap sm{T, W, (int64_t)a.weight_odd};
        t0 = sm.start(j);
        t1 = sm.start(j + 1);
    } else {
        wave_slice(a, T, j, t0, t1);
    }
    if (t0 >= t1) return;
    const int n = (int)(t1 - t0);
    const int gq = lane & 15, quad = lane >> 4;
    const int G = a.heads_per_unit;
    // Padded head slots (gq >= G) reuse head G-1's query: their score and value columns
    // are computed and never written.  (Zeroing them would need a wait on the query
    // load right where it is issued, draining the K/V prefetch.)
    const int gqc = min(gq, G - 1);
    const int64_t blk_stride = (int64_t)a.num_kv_heads * TILE;
    // Block size >= 16: K load kk of lane l is chunk 4*kk + l/16 of token l%16 of the tile
    // (1 KiB contiguous per load instruction); V^T load mt of lane l is dim 16*mt + l%16,
    // tokens 4*(l/16)..+3 (512 bytes contiguous).  Block size 1: whole rows (below).
    const int voff = gq * 4 + quad;
    const uint16_t* kpool = static_cast<const uint16_t*>(a.k_pool);
    const uint16_t* vpool = static_cast<const uint16_t*>(a.v_pool);
    uint16_t* vrows = s_vt + (threadIdx.x >> 6) * kTile * LDW;
    uint16_t* krows = s_kt + (threadIdx.x >> 6) * kTile * LDW;

    Cursor lc = locate(a, s_pref, t0);   // tile being loaded (one ahead)
    Cursor cc = lc;                       // tile being computed

    kvec qop[KI];
    auto load_q = [&](const Cursor& c) __attribute__((always_inline)) {
        const uint16_t* qh = static_cast<const uint16_t*>(a.q) +
                             ((int64_t)c.s * a.num_q_heads + c.u * G + gqc) * D + 8 * quad;
#pragma unroll
        for (int kk = 0; kk < KI; ++kk)
            qop[kk] = __builtin_bit_cast(kvec, *reinterpret_cast<const i32x4*>(qh + 32 * kk));
    };
    // Block size 1: lane l's id is that of token l % 16 of the tile (tokens at or past ctx
    // take token ctx - 1's), read with a vector load one step before the tile's rows are
    // loaded: `ic` is the cursor of the tile whose ids are in flight, `ahead` its index in
    // the slice (at the slice's end the last tile's ids are read again, so every step
    // issues the same loads).  Issued ahead of the previous tile's rows, the ids are waited
    // for without waiting for those rows.
    Cursor ic = lc;
    int ahead = 0;
    int32_t id_next = 0;
    auto fetch_ids = [&](const Cursor& c) __attribute__((always_inline)) {
        return a.block_tables[(int64_t)c.s * a.max_blocks_per_seq +
                              min(kTile * c.it + (lane & 15), c.ctx - 1)];
    };
    auto next_ids = [&]() __attribute__((always_inline)) {
        if (ahead + 1 < n) {
            advance(a, ic);
            ++ahead;
        }
        id_next = fetch_ids(ic);
    };
    auto load_kv = [&](const Cursor& c, int32_t raw, i32x4 (&kr)[KI], vbuf& vr, bool& bad) __attribute__((always_inline)) {
        if constexpr (BS == 1) {
            // whole rows: load i of lane l is chunk l % (D / 8) of token (512 / D) i + l / (D / 8);
            // an id outside [0, num_blocks) reads block 0 and flags the unit
            const bool oob = (uint32_t)raw >= (uint32_t)a.num_blocks;
            bad = __ballot(oob) != 0;
            const int32_t idv = oob ? 0 : raw;
#pragma unroll
            for (int i = 0; i < KI; ++i) {
                const int64_t base = load_id_bs1<D>(idv, i, lane) * blk_stride + (int64_t)c.u * D;
                kr[i] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(kpool + base) + lane % (D / 8));
                vr[i] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(vpool + base) + lane % (D / 8));
            }
        } else {
            const int32_t bid = tile_block<BS>(a, c, bad);
            const int64_t base = (int64_t)c.u * TILE + bid * blk_stride + (c.it & (TPB - 1)) * (kTile * D);
            const i32x4* kt = reinterpret_cast<const i32x4*>(kpool + base) + lane;
            const i32x2* vt = reinterpret_cast<const i32x2*>(vpool + base) + voff;
#pragma unroll
            for (int kk = 0; kk < KI; ++kk) kr[kk] = __builtin_nontemporal_load(kt + kk * 64);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) vr[mt] = __builtin_nontemporal_load(vt + mt * 64);
        }
    };

    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m = kNegInf, lsum = 0.f;
    bool unit_bad = false;
    bool first_here = PM ? cc.it % a.pm_tiles == 0 : cc.it == 0;
    Pending pend;

    // PM: finished pieces wait in the wave's LDS region (G x D values, then G maxima, G
    // sums, the first row and a flags word) and go to memory together at the end of the
    // slice, so that no store sits between a tile's loads and the wait for them (stores
    // every partition measured 0.62 of peak against 0.77 without).  A slice with more
    // pieces than the region holds stores the rest directly.
    const int pm_piece = (G * (D + 2) + 2 + 3) & ~3;         // floats per piece (16-byte aligned)
    const int pm_cap = PM ? kPmWaveFloats<BS>() / pm_piece : 0;
    float* pm_lds = s_pm + (threadIdx.x >> 6) * kPmWaveFloats<BS>();
    int pm_count = 0;
    const int64_t pm_stride = 2 * (int64_t)a.pm_max_parts;  // rows between query heads
    auto capture = [&](const Cursor& c) __attribute__((always_inline)) {
        const float lw = sum_across_quads(lsum);
        const int p = c.it / a.pm_tiles;
        const bool has_end = (c.it + 1) % a.pm_tiles == 0 || c.it == c.nt - 1;
        // row of query head 0 of the unit; head h adds h * pm_stride
        const int64_t row0 = ((int64_t)c.s * a.num_q_heads + c.u * G) * pm_stride + 2 * p;
        const int kk = first_here ? 0 : 1;
        const bool mark = first_here && has_end;            // not cut: the second row is empty
        if (pm_count < pm_cap) {
            float* pc = pm_lds + pm_count * pm_piece;
            if (gq < G) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    *reinterpret_cast<f32x4*>(pc + gq * D + 16 * mt + 4 * quad) =
                        unit_bad ? (f32x4){NAN, NAN, NAN, NAN} : acc[mt];
                if (quad == 0) {
                    pc[G * D + gq] = unit_bad ? NAN : m;
                    pc[G * D + G + gq] = unit_bad ? NAN : lw;
                }
            }
            if (lane == 0) {
                reinterpret_cast<int*>(pc)[G * (D + 2)] = (int)(row0 + kk);   // (fits: checked on the host)
                reinterpret_cast<int*>(pc)[G * (D + 2) + 1] = mark ? 1 : 0;
            }
            ++pm_count;
        } else if (gq < G) {
            const int64_t row = row0 + gq * pm_stride + kk;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                *reinterpret_cast<f32x4*>(a.pm_acc + row * D + 16 * mt + 4 * quad) =
                    unit_bad ? (f32x4){NAN, NAN, NAN, NAN} : acc[mt];
            if (quad == 0) {
                a.pm_m[row] = unit_bad ? NAN : m;
                a.pm_l[row] = unit_bad ? NAN : lw;
                if (mark) a.pm_m[row + 1] = kNegInf;
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
        m = kNegInf;
        lsum = 0.f;
        unit_bad = false;
        first_here = true;
    };
    // the pieces held in LDS to memory: per piece, the G x D values 4 to a lane, then the
    // maxima and sums (lane h < G), and the empty second rows of partitions not cut
    auto store_pieces = [&]() __attribute__((always_inline)) {
        for (int k = 0; k < pm_count; ++k) {
            const float* pc = pm_lds + k * pm_piece;
            const int64_t row_h0 = uni(reinterpret_cast<const int*>(pc)[G * (D + 2)]);
            const int mark = uni(reinterpret_cast<const int*>(pc)[G * (D + 2) + 1]);
            for (int i = 4 * lane; i < G * D; i += 256) {
                const int h = i / D, d = i - h * D;
                *reinterpret_cast<f32x4*>(a.pm_acc + (row_h0 + h * pm_stride) * D + d) =
                    *reinterpret_cast<const f32x4*>(pc + i);
            }
            if (lane < G) {
                const int64_t row = row_h0 + lane * pm_stride;
                a.pm_m[row] = pc[G * D + lane];
                a.pm_l[row] = pc[G * D + G + lane];
                if (mark) a.pm_m[row + 1] = kNegInf;
            }
        }
    };

    // Write the finished (or slice-cut) unit of cursor c, then reset the state.
    auto finish = [&](const Cursor& c) __attribute__((always_inline)) {
        const bool direct = first_here && c.it == c.nt - 1;
        const float lw = sum_across_quads(lsum);
        const int q = c.s * a.units + c.u;
        if (gq < G) {
            if (direct) {
                const int64_t ob = ((int64_t)c.s * a.num_q_heads + c.u * G + gq) * D;
                const float inv = 1.f / lw;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        store_out<OUT_DT>(a.out, ob + 16 * mt + 4 * quad + r,
                                          unit_bad ? NAN : acc[mt][r] * inv);
            } else {
                const int64_t piece = ((int64_t)j + q) * G + gq;
                // the unit's G x D piece is one contiguous region: 16-byte stores, each
                // head row written as 64-byte runs
                float* region = a.ws_acc + ((int64_t)j + q) * G * D;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    put_coherent4(region, (uint32_t)(G * D * 4),
                                  (uint32_t)((gq * D + 16 * mt + 4 * quad) * 4),
                                  unit_bad ? (f32x4){NAN, NAN, NAN, NAN} : acc[mt]);
                if (quad == 0) {
                    put_coherent(a.ws_m + piece, unit_bad ? NAN : m);
                    put_coherent(a.ws_l + piece, unit_bad ? NAN : lw);
                }
            }
        }
        if (!direct) pend.add(c.s, c.u, c.nt);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
        m = kNegInf;
        lsum = 0.f;
        unit_bad = false;
        first_here = true;
    };

    // Compute the tile of cc from registers kr/vr.  If the next tile (nc) starts a new
    // unit, its queries are loaded into qop once the score MFMAs have read them.
    auto compute = [&](i32x4 (&kr)[KI], vbuf& vin, bool bad, bool next_unit,
                       const Cursor& nc) __attribute__((always_inline)) {
        i32x2 vr[MT];
        if constexpr (BS == 1) {
            // K back in the score product's operand layout (token l % 16, dims 32 kk +
            // 8 (l / 16) ..), V transposed (4 tokens of one dim per lane)
            lds_put_whole_rows<D, KI>(krows, LDW, lane, kr);
            lds_put_whole_rows<D, KI>(vrows, LDW, lane, vin);
#pragma unroll
            for (int kk = 0; kk < KI; ++kk)
                kr[kk] = *reinterpret_cast<const i32x4*>(krows + (lane & 15) * LDW + 32 * kk + 8 * (lane >> 4));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                uint32_t e[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) e[jj] = vrows[(4 * quad + jj) * LDW + 16 * mt + gq];
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
        if (next_unit) load_q(nc);
        const int valid = min(kTile, cc.ctx - cc.it * kTile);   // tokens of this tile in the context
        const int tok0 = 4 * quad;
        float x[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) x[jj] = (tok0 + jj < valid) ? sc[jj] * a.scale_log2 : kNegInf;
        const float xm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        if (__ballot(xm > m + kRescaleSlack)) {
            const float mnew = fmaxf(m, max_across_quads(xm));
            const float alpha = exp2_fast(m - mnew);
            lsum *= alpha;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
            m = mnew;
        }
        s16x4 phi, plo;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float pf = exp2_fast(x[jj] - m);
            const uint16_t hi = f32_to_bits16<DT>(pf);
            const uint16_t lo = f32_to_bits16<DT>(pf - bits_to_f32<DT>(hi));
            phi[jj] = (short)hi;
            plo[jj] = (short)lo;
            lsum += pf;
        }
        if (valid < kTile) {
            // slots past the context may hold anything (NaN included): clear them
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                uint32_t lo = (uint32_t)vr[mt][0], hi = (uint32_t)vr[mt][1];
                if (tok0 + 0 >= valid) lo &= 0xFFFF0000u;
                if (tok0 + 1 >= valid) lo &= 0x0000FFFFu;
                if (tok0 + 2 >= valid) hi &= 0xFFFF0000u;
                if (tok0 + 3 >= valid) hi &= 0x0000FFFFu;
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
        unit_bad |= bad;
    };

    // Ring of R tile buffers: while tile k is computed, tiles k+1 .. k+R-1 are in flight.
    constexpr int R = stream_depth<D>();
    i32x4 kbuf[R][KI];
    vbuf vbufs[R];
    bool bbuf[R];
#pragma unroll
    for (int r = 0; r < R; ++r) bbuf[r] = false;

    int done = 0;
    // Waves with more of their slice left get issue priority: co-resident waves share
    // the CU's memory pipe unevenly (oldest first), and a slice split is only balanced
    // if the waves progress together.
    auto prio = [&]() __attribute__((always_inline)) {
        const int pr = ((n - done) * 4) / (n + 1);
        if (pr >= 3) __builtin_amdgcn_s_setprio(3);
        else if (pr == 2) __builtin_amdgcn_s_setprio(2);
        else if (pr == 1) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
        ++done;
    };
    // load the tile after the last one loaded into slot sl
    auto produce = [&](int sl) __attribute__((always_inline)) {
        advance(a, lc);
        if constexpr (BS == 1) {
            const int32_t raw = id_next;   // lc's ids (ic is lc here)
            next_ids();
            __builtin_amdgcn_sched_barrier(0);
            load_kv(lc, raw, kbuf[sl], vbufs[sl], bbuf[sl]);
        } else {
            load_kv(lc, 0, kbuf[sl], vbufs[sl], bbuf[sl]);
        }
        // Keep these loads ahead of everything that waits on the tile about to be
        // computed: left alone, the scheduler hoists the first score product (and with
        // it a wait on that tile's loads) into the block-id lookup's latency, which
        // leaves one tile fewer in flight.
        __builtin_amdgcn_sched_barrier(0);
    };
    // compute the tile of cursor cc from slot sl, then move cc on (if a tile follows)
    auto consume = [&](int sl, bool has_next) __attribute__((always_inline)) {
        Cursor nc = cc;
        bool next_unit = false, flush = false;
        if (has_next) {
            advance(a, nc);
            next_unit = nc.s != cc.s || nc.u != cc.u;
            flush = next_unit || (PM && nc.it % a.pm_tiles == 0);
        }
        compute(kbuf[sl], vbufs[sl], bbuf[sl], next_unit, nc);
        if (flush) {
            if constexpr (PM) capture(cc);
            else finish(cc);
        }
        cc = nc;
    };

    load_q(cc);
    if constexpr (BS == 1) {
        const int32_t raw = fetch_ids(lc);
        next_ids();
        load_kv(lc, raw, kbuf[0], vbufs[0], bbuf[0]);
    } else {
        load_kv(lc, 0, kbuf[0], vbufs[0], bbuf[0]);
    }
    if (n >= 2 * R - 1) {
        // Every step of the main loop loads one tile and computes one, so the number
        // of loads in flight is the same on every path and the compiler waits for
        // exactly the tile being computed.
#pragma unroll
        for (int r = 1; r < R - 1; ++r) produce(r);
        const int loading = n - (R - 1);   // steps that also load a tile
        int k = 0;
        for (; k + R <= loading; k += R) {
#pragma unroll
            for (int j = 0; j < R; ++j) {
                prio();
                produce((j + R - 1) % R);
                consume(j, true);
            }
        }
        // fewer than R loading steps left, then R - 1 tiles to compute; k % R == 0
#pragma unroll
        for (int j = 0; j < 2 * R - 2; ++j) {
            if (k + j < n) {
                prio();
                if (k + j < loading) produce((j + R - 1) % R);
                consume(j % R, k + j + 1 < n);
            }
        }
    } else {
        // short slice: two buffers
#pragma unroll
        for (int j = 0; j < 2 * R - 2; ++j) {
            if (j < n) {
                prio();
                if (j + 1 < n) produce((j + 1) % 2);
                consume(j % 2, j + 1 < n);
            }
        }
    }
    if constexpr (PM) {
        capture(cc);
        store_pieces();
    } else {
        finish(cc);
    }
    __builtin_amdgcn_s_setprio(0);
    if constexpr (!PM) publish_pieces<D, OUT_DT, 8, (D == 64 ? 8 : 4)>(a, s_pref, pend, T, lane);
}

// ---------------------------------------------------------------------------------
// VALU stream-K kernel: unit = one query head (a group of 1, or fp32).  The per-tile
// math is the fixed-partition VALU kernel's.
// ---------------------------------------------------------------------------------
template <int D, int DT, int OUT_DT, int BS>
__global__ __launch_bounds__(kWaves * 64)
__attribute__((amdgpu_waves_per_eu(valu_waves_per_simd<D, DT == DT_F32 ? 4 : 2, true>())))
void attn_valu_streamk(StreamArgs a) {
    using bits_t = typename std::conditional<DT == DT_F32, uint32_t, uint16_t>::type;
    constexpr int E = sizeof(bits_t);
    constexpr int X = 16 / E;
    constexpr int NI = kTile * D * E / 1024;
    constexpr int TILE = BS * D;
    constexpr int TPB = BS >= kTile ? BS / kTile : 1;
    constexpr int LDW = D + X;
    __shared__ bits_t s_vt[BS == 1 ? kWaves * kTile * LDW : 1];

    extern __shared__ int s_pref[];
    const int tiles_per_unit = build_prefix(a, s_pref);
    nan_invalid_sequences<D, OUT_DT>(a, s_pref);
    const int lane = threadIdx.x & 63;
    const int j = uni(blockIdx.x * kWaves + (threadIdx.x >> 6));
    if (j >= a.waves) return;
    const int64_t T = (int64_t)a.units * tiles_per_unit;
    int64_t t0, t1;
    wave_slice(a, T, j, t0, t1);
    if (t0 >= t1) return;
    const int n = (int)(t1 - t0);
    const int tok = lane & 15, kq = lane >> 4, vpiece = lane % E;
    const int64_t blk_stride = (int64_t)a.num_kv_heads * TILE;
    // K: load i of lane l is chunk 4*i + l/16 of token l%16; V (dim-major): load i is
    // dim (64*i + l)/E, tokens X*(l%E)..+X
    const bits_t* kpool = static_cast<const bits_t*>(a.k_pool);
    const bits_t* vpool = static_cast<const bits_t*>(a.v_pool);
    bits_t* vrows = s_vt + (threadIdx.x >> 6) * kTile * LDW;

    Cursor lc = locate(a, s_pref, t0);
    Cursor cc = lc;

    // query: raw bits of the lane's D/4 dims (chunks 4*i + kq), converted on unit change
    i32x4 qraw[NI];
    float qr[NI][X];
    auto load_q = [&](const Cursor& c) __attribute__((always_inline)) {
        const i32x4* qh = reinterpret_cast<const i32x4*>(
            static_cast<const bits_t*>(a.q) + ((int64_t)c.s * a.num_q_heads + c.u) * D);
#pragma unroll
        for (int i = 0; i < NI; ++i) qraw[i] = qh[4 * i + kq];
    };
    auto convert_q = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            bits_t qb[X];
            __builtin_memcpy(qb, &qraw[i], 16);
#pragma unroll
            for (int e = 0; e < X; ++e) qr[i][e] = bits_to_f32<DT>(qb[e]) * a.scale_log2;
        }
    };
    auto load_kv = [&](const Cursor& c, i32x4 (&kr)[NI], i32x4 (&vr)[NI], bool& bad) __attribute__((always_inline)) {
        if constexpr (BS == 1) {
            const int32_t bid = lane_block_bs1(a.block_tables + (int64_t)c.s * a.max_blocks_per_seq,
                                               c.it, c.ctx, a.num_blocks, lane, bad);
            const int64_t base = bid * blk_stride + (int64_t)(c.u / a.group) * D;
            const i32x4* kt = reinterpret_cast<const i32x4*>(kpool + base) + kq;
            const i32x4* vt = reinterpret_cast<const i32x4*>(vpool + base) + kq;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                kr[i] = __builtin_nontemporal_load(kt + 4 * i);
                vr[i] = __builtin_nontemporal_load(vt + 4 * i);
            }
        } else {
            const int32_t bid = tile_block<BS>(a, c, bad);
            const int64_t base = (int64_t)(c.u / a.group) * TILE + bid * blk_stride +
                                 (c.it & (TPB - 1)) * (kTile * D);
            const i32x4* kt = reinterpret_cast<const i32x4*>(kpool + base) + lane;
            const i32x4* vt = reinterpret_cast<const i32x4*>(vpool + base) + lane;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                kr[i] = __builtin_nontemporal_load(kt + i * 64);
                vr[i] = __builtin_nontemporal_load(vt + i * 64);
            }
        }
    };

    float acc[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) acc[i] = 0.f;
    float m = kNegInf, lsum = 0.f;
    bool unit_bad = false;
    bool first_here = cc.it == 0;
    bool q_stale = false;    // qraw holds the next unit's query, not yet converted
    Pending pend;

    auto finish = [&](const Cursor& c) __attribute__((always_inline)) {
        const bool direct = first_here && c.it == c.nt - 1;
        float lw = lsum;
        lw += __shfl_xor(lw, 1);
        lw += __shfl_xor(lw, 2);
        lw += __shfl_xor(lw, 4);
        lw += __shfl_xor(lw, 8);
        float rows[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            float r = acc[i];
            if constexpr (E >= 2) r += __shfl_xor(r, 1);
            if constexpr (E >= 4) r += __shfl_xor(r, 2);
            rows[i] = r;
        }
        const int q = c.s * a.units + c.u;
        if (vpiece == 0) {
            if (direct) {
                const int64_t ob = ((int64_t)c.s * a.num_q_heads + c.u) * D;
                const float inv = 1.f / lw;
#pragma unroll
                for (int i = 0; i < NI; ++i)
                    store_out<OUT_DT>(a.out, ob + (64 * i + lane) / E, unit_bad ? NAN : rows[i] * inv);
            } else {
                const int64_t piece = (int64_t)j + q;
#pragma unroll
                for (int i = 0; i < NI; ++i)
                    put_coherent(a.ws_acc + piece * D + (64 * i + lane) / E, unit_bad ? NAN : rows[i]);
                if (lane == 0) {
                    put_coherent(a.ws_m + piece, unit_bad ? NAN : m);
                    put_coherent(a.ws_l + piece, unit_bad ? NAN : lw);
                }
            }
        }
        if (!direct) pend.add(c.s, c.u, c.nt);
#pragma unroll
        for (int i = 0; i < NI; ++i) acc[i] = 0.f;
        m = kNegInf;
        lsum = 0.f;
        unit_bad = false;
        first_here = true;
    };

    auto compute = [&](i32x4 (&kr)[NI], i32x4 (&vin)[NI], bool bad, bool next_unit,
                       const Cursor& nc) __attribute__((always_inline)) {
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
        if (q_stale) {
            convert_q();
            q_stale = false;
        }
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            bits_t kb[X];
            __builtin_memcpy(kb, &kr[i], 16);
#pragma unroll
            for (int e = 0; e < X; ++e) part = fmaf(qr[i][e], bits_to_f32<DT>(kb[e]), part);
        }
        if (next_unit) {
            load_q(nc);
            q_stale = true;
        }
        const float sc = sum_across_quads(part);
        const int valid = min(kTile, cc.ctx - cc.it * kTile);
        const float x = tok < valid ? sc : kNegInf;
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
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            bits_t vb[X];
            __builtin_memcpy(vb, &vr[i], 16);
            float r = acc[i];
#pragma unroll
            for (int e = 0; e < X; ++e) {
                const float v = (vpiece * X + e < valid) ? bits_to_f32<DT>(vb[e]) : 0.f;
                r = fmaf(pw[e], v, r);
            }
            acc[i] = r;
        }
        unit_bad |= bad;
    };

    i32x4 kA[NI], kB[NI], vA[NI], vB[NI];
    bool bA = false, bB = false;
    int done = 0;
    auto step = [&](i32x4 (&kc)[NI], i32x4 (&vc)[NI], bool bc, i32x4 (&kn)[NI],
                    i32x4 (&vn)[NI], bool& bn) __attribute__((always_inline)) {
        // issue priority to the waves with more of their slice left (see the MFMA kernel)
        {
            const int pr = ((n - done) * 4) / (n + 1);
            if (pr >= 3) __builtin_amdgcn_s_setprio(3);
            else if (pr == 2) __builtin_amdgcn_s_setprio(2);
            else if (pr == 1) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
            ++done;
        }
        advance(a, lc);
        load_kv(lc, kn, vn, bn);
        // Keep the next tile's loads ahead of everything that waits on the current one:
        // left alone, the scheduler hoists the first score product (and with it a wait
        // on the current tile's loads) into the block-id lookup's latency, which leaves
        // one tile in flight instead of two.
        __builtin_amdgcn_sched_barrier(0);
        const bool next_unit = lc.s != cc.s || lc.u != cc.u;
        compute(kc, vc, bc, next_unit, lc);
        if (next_unit) finish(cc);
        cc = lc;
    };

    load_q(cc);
    q_stale = true;
    load_kv(lc, kA, vA, bA);
    int k = 0;
    for (; k + 2 < n; k += 2) {
        step(kA, vA, bA, kB, vB, bB);
        step(kB, vB, bB, kA, vA, bA);
    }
    if (k + 1 < n) {
        step(kA, vA, bA, kB, vB, bB);
        compute(kB, vB, bB, false, cc);
    } else {
        compute(kA, vA, bA, false, cc);
    }
    finish(cc);
    __builtin_amdgcn_s_setprio(0);
    publish_pieces<D, OUT_DT, 1, 8>(a, s_pref, pend, T, lane);
}

// ---------------------------------------------------------------------------------
// Merge.  Units that one wave covered entirely were written by that wave; the others
// combine their pieces in slice order:
// out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p, M = max_p m_p.
// ---------------------------------------------------------------------------------
StreamArgs make_args(const pkv::StreamLaunch& L, const pkv::StreamPlan& P) {
    StreamArgs a;
    a.out = L.out;
    a.q = L.q;
    a.k_pool = L.k_pool;
    a.v_pool = L.v_pool;
    a.block_tables = L.block_tables;
    a.context_lens = L.context_lens;
    a.counters = L.counters;
    a.ws_m = reinterpret_cast<float*>(L.data);
    a.ws_l = reinterpret_cast<float*>(L.data + (P.l_off - P.m_off));
    a.ws_acc = reinterpret_cast<float*>(L.data + (P.acc_off - P.m_off));
    a.num_seqs = L.num_seqs;
    a.max_blocks_per_seq = L.max_blocks_per_seq;
    a.num_q_heads = L.num_q_heads;
    a.num_kv_heads = L.num_kv_heads;
    a.group = L.num_q_heads / L.num_kv_heads;
    a.units = P.units;
    a.heads_per_unit = P.heads_per_unit;
    a.num_blocks = L.num_blocks;
    a.max_context_len = L.max_context_len;
    a.waves = P.waves;
    // XCD-weighted slices where they measured faster (one wave per SIMD: head_dim 128
    // and up; 16- or 32-token blocks): 0.744 against 0.735 of peak on the GQA workload,
    // 0.793 against 0.781 on the MHA one; at head_dim 64 and block size 1 equal slices
    // were faster (0.677 against 0.663, 0.571 against 0.557).  The weights were measured
    // on MI355X in SPX mode (256 compute units, workgroup b on die b % 8); any other
    // device shape gets equal slices.
    a.weight_odd = (L.head_dim >= 128 && L.block_size >= 16 && pkv::device_shape().mi355x_spx)
                       ? 58 : (int32_t)kWeightEven;
    a.scale_log2 = L.scale * kLog2e;
    a.pm_tiles = L.pm_tiles;
    a.pm_max_parts = L.pm_max_parts;
    a.pm_m = L.pm_m;
    a.pm_l = L.pm_l;
    a.pm_acc = L.pm_acc;
    return a;
}

template <int D, int DT, int OUT, int BS>
void launch_part_t(const StreamArgs& a, bool mfma, hipStream_t st) {
    const dim3 grid((unsigned)((a.waves + kWaves - 1) / kWaves));
    const size_t lds = (size_t)(a.num_seqs + 1) * sizeof(int);
    if constexpr (DT == DT_F32) {
        attn_valu_streamk<D, DT, OUT, BS><<<grid, dim3(kWaves * 64), lds, st>>>(a);
    } else {
        if (mfma && a.pm_tiles > 0) attn_mfma_streamk<D, DT, OUT, BS, true><<<grid, dim3(kWaves * 64), lds, st>>>(a);
        else if (mfma) attn_mfma_streamk<D, DT, OUT, BS, false><<<grid, dim3(kWaves * 64), lds, st>>>(a);
        else attn_valu_streamk<D, DT, OUT, BS><<<grid, dim3(kWaves * 64), lds, st>>>(a);
    }
}

template <int D, int DT, int BS>
void launch_part_d(const StreamArgs& a, int out_dtype, bool mfma, hipStream_t st) {
    if (out_dtype == PAGED_KV_F32) launch_part_t<D, DT, DT_F32, BS>(a, mfma, st);
    else launch_part_t<D, DT, DT, BS>(a, mfma, st);
}

template <int D, int BS>
void launch_part_dd(const StreamArgs& a, int dtype, int out_dtype, bool mfma, hipStream_t st) {
    switch (dtype) {
        case PAGED_KV_F32: launch_part_d<D, DT_F32, BS>(a, out_dtype, mfma, st); break;
        case PAGED_KV_F16: launch_part_d<D, DT_F16, BS>(a, out_dtype, mfma, st); break;
        default: launch_part_d<D, DT_BF16, BS>(a, out_dtype, mfma, st); break;
    }
}

template <int D>
void launch_part_b(const StreamArgs& a, int block_size, int dtype, int out_dtype, bool mfma,
                   hipStream_t st) {
    switch (block_size) {
        case 1: launch_part_dd<D, 1>(a, dtype, out_dtype, mfma, st); break;
        case 32: launch_part_dd<D, 32>(a, dtype, out_dtype, mfma, st); break;
        default: launch_part_dd<D, 16>(a, dtype, out_dtype, mfma, st); break;
    }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

namespace pkv {

StreamPlan stream_plan(int32_t num_seqs, int32_t hq, int32_t hkv, int32_t dtype, int32_t head_dim,
                       int32_t max_ctx, bool* ok) {
    StreamPlan p{};
    *ok = num_seqs >= 0 && num_seqs <= kStreamMaxSeqs && hq >= 1 && hkv >= 1 && hq % hkv == 0 &&
          max_ctx >= 1 && head_dim >= 1;
    if (!*ok) return p;
    const int group = hq / hkv;
    p.mfma = dtype != PAGED_KV_F32 && group >= 2;
    p.units = p.mfma ? hkv : hq;
    p.heads_per_unit = p.mfma ? group : 1;
    const int64_t max_tiles = (int64_t)((max_ctx + kTile - 1) / kTile) * num_seqs * p.units;
    // at least kStreamMinSlice tiles per wave (on the bound max_tiles): thinner slices cut
    // every unit into many pieces, and the merge's round trips grow with their number
    p.waves = (int32_t)std::max<int64_t>(
        1, std::min<int64_t>(stream_max_waves(device_shape().compute_units, head_dim,
                                              elem_bytes(dtype), p.mfma),
                             (max_tiles + kStreamMinSlice - 1) / kStreamMinSlice));
    p.max_pieces = (int64_t)p.waves + (int64_t)num_seqs * p.units;
    const size_t rows = (size_t)p.max_pieces * p.heads_per_unit;
    // the counters come first, so that a call with no more (sequence, unit) counters
    // than an earlier one on the same workspace finds them at zero
    p.cnt_off = 0;
    p.m_off = align256((size_t)num_seqs * p.units * sizeof(int32_t));
    p.l_off = p.m_off + align256(rows * sizeof(float));
    p.acc_off = p.l_off + align256(rows * sizeof(float));
    p.ws_bytes = p.acc_off + rows * head_dim * sizeof(float);
    return p;
}

void launch_streamk_partition(const StreamLaunch& L, const StreamPlan& P, void* stream) {
    const StreamArgs a = make_args(L, P);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    switch (L.head_dim) {
        case 64: launch_part_b<64>(a, L.block_size, L.dtype, L.out_dtype, P.mfma, st); break;
        case 256: launch_part_b<256>(a, L.block_size, L.dtype, L.out_dtype, P.mfma, st); break;
        default: launch_part_b<128>(a, L.block_size, L.dtype, L.out_dtype, P.mfma, st); break;
    }
}

}  // namespace pkv
