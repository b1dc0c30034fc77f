// prune.hip -- in-place drop / regrow of connections with nnz fixed.
//
// The DST update of the "Padded-CSR" post (section 4.3: drop a fraction of the
// live entries, grow the same number elsewhere) applied in place on the COO
// triple as in the SNACK paper's Figure 1, with the SET-style rule:
//   drop   the n_drop entries of smallest |v|, in the total order of the key
//          (IEEE bits of |v|, canonical slot) -- found by an MSB-first radix
//          select over the magnitude bits plus a slot-order scan of the ties;
//   grow   n_drop positions uniform over the cells empty after the drop, value
//          +0.0: candidate t is SplitMix64 output number epoch*2^40 + t of the
//          generator seeded with the layer seed (Steele, Lea & Flood 2014),
//          mapped onto [0, M*K) by the high word of the 64x64 product; a
//          candidate is accepted if its cell is neither kept nor accepted at a
//          smaller t.
// Occupancy lives in two bitmaps over the M*K cells: `kept` and `occ` (kept or
// grown).  Candidates are tested in batches against `occ`; the free ones claim
// their cell in `occ` with an atomic OR, and the rare cells claimed twice in a
// batch are resolved in an open-addressing table that keeps the smallest
// candidate index per cell (an atomic minimum on (cell, index) packed in one
// word, so the order of the atomics does not matter).  A scan in t order
// keeps the first `need` accepted and the rest give their cells back -- the
// result never depends on the batch size.  The new canonical order is then the set bits of `occ` in
// ascending position: prefix counts of bits place every entry, and a kept
// cell takes the next kept value (its rank in `kept`).
// Every step is integer work and deterministic.
#include <algorithm>
#include <cmath>

#include "internal.h"

namespace snack {
namespace {

constexpr int kThreads = 256;
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr int64_t kMaxBatch = 1 << 21;          // candidates per batch
constexpr uint64_t kEmpty = ~0ull;              // empty table word
constexpr uint64_t kMaxBitmapBits = 1ull << 34;


inline unsigned grid_for(int64_t n)
{
    int64_t g = (n + kThreads - 1) / kThreads;
    if (g < 1) g = 1;
    if (g > 65535LL * 8) g = 65535LL * 8;
    return (unsigned)g;
}

inline size_t al(size_t b) { return (b + 255) & ~(size_t)255; }

__device__ inline uint64_t splitmix64_output(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ inline uint32_t mag_bits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// inclusive sum over lanes 0 .. lane: shifts by 1, 2, 4, 8 inside each row of
// 16 lanes (DPP row_shr, zero where the source lies before the row), then the
// end of row 0 added to row 1 and of row 2 to row 3 (row_bcast:15), then the
// end of row 1 to rows 2 and 3 (row_bcast:31); no LDS round trips
__device__ inline int32_t wave_incl(int32_t v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
    return v;
}

// the wavefront's sum (uniform)
__device__ inline int32_t wave_sum(int32_t v) { return __builtin_amdgcn_readlane(wave_incl(v), kWave - 1); }

// ---- drop: radix select ---------------------------------------------------
// Four passes over the magnitude keys, eight bits each, most significant
// first.  state: [0] the n_drop-th smallest key T, [1] its rank among the keys
// equal to T, [2] the number of keys equal to T (all three written after the
// last pass); [3 + 3j .. 5 + 3j] the prefix, rank and count after pass j's pick.
// Pass j writes histogram set j; the digit of pass j is picked by every
// workgroup of the next kernel from set j (no separate launch), and workgroup 0
// records it in its own state slot, which no workgroup of that kernel reads.
// Each thread takes sixteen consecutive keys (four 16-byte loads) and adds runs
// of equal digits before touching LDS, which keeps the first passes (where
// nearly every key shares a digit) free of contention; each workgroup adds its
// nonzero bins to one of kSelCopies copies (atomics on one address serialise).
constexpr int kSelThreads = 256;
constexpr int kSelPer = 16;
constexpr int kSelCopies = 32;
constexpr int kSelPasses = 4;
constexpr int kSelHist = kSelCopies * 256;   // words of one pass's histograms

__global__ void prune_init_kernel(uint32_t* __restrict__ state, uint32_t* __restrict__ hist, uint32_t rank0,
                                  int32_t* __restrict__ fill, int32_t nfill)
{
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (int64_t i = i0; i < (int64_t)kSelPasses * kSelHist; i += (int64_t)gridDim.x * blockDim.x) hist[i] = 0u;
    for (int64_t i = i0; i < nfill; i += (int64_t)gridDim.x * blockDim.x) fill[i] = 0;
    if (i0 < 16) state[i0] = i0 == 1 ? rank0 : 0u;
}

struct SelPick {
    uint32_t prefix, rank, equal;
};

// The digit (at `shift`) holding rank `rank` among the keys that match
// `prefix`, from the histograms of the pass that counted them: the first digit
// whose running count passes the rank (the last digit if none does).  Called
// by every thread of a 256-thread workgroup.
__device__ inline SelPick sel_pick(const uint32_t* __restrict__ hist, uint32_t prefix, uint32_t rank, int shift)
{
    __shared__ uint32_t s_red[256 / kWave];
    __shared__ SelPick s_pick;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
    uint32_t t = 0;
#pragma unroll
    for (int c = 0; c < kSelCopies; ++c) t += hist[c * 256 + tid];
    const uint32_t inc = (uint32_t)wave_incl((int32_t)t);
    if (lane == kWave - 1) s_red[w] = inc;
    __syncthreads();
    uint32_t ex = inc - t;
    for (int i = 0; i < w; ++i) ex += s_red[i];
    if ((rank >= ex && rank < ex + t) || (tid == 255 && rank >= ex + t)) {
        s_pick.prefix = prefix | ((uint32_t)tid << shift);
        s_pick.rank = rank - ex;
        s_pick.equal = t;
    }
    __syncthreads();
    return s_pick;
}

template <int PASS>
__global__ void __launch_bounds__(kSelThreads) sel_pass_kernel(const float* __restrict__ vals, int64_t n,
                                                               uint32_t* __restrict__ state,
                                                               uint32_t* __restrict__ hist)
{
    constexpr int shift = 24 - 8 * PASS;
    __shared__ uint32_t h[256];
    const int tid = threadIdx.x;
    h[tid] = 0;
    uint32_t prefix = 0;
    if constexpr (PASS > 0) {
        const uint32_t p0 = PASS == 1 ? 0u : state[3 + 3 * (PASS - 2)];
        const uint32_t r0 = PASS == 1 ? state[1] : state[4 + 3 * (PASS - 2)];
        const SelPick pk = sel_pick(hist + (PASS - 1) * kSelHist, p0, r0, shift + 8);
        if (blockIdx.x == 0 && tid == 0) {
            state[3 + 3 * (PASS - 1)] = pk.prefix;
            state[4 + 3 * (PASS - 1)] = pk.rank;
            state[5 + 3 * (PASS - 1)] = pk.equal;
        }
        prefix = pk.prefix;
    }
    __syncthreads();
    const uint32_t hi_mask = PASS == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    const int64_t k0 = ((int64_t)blockIdx.x * kSelThreads + tid) * kSelPer;
    uint32_t key[kSelPer];
    if (k0 + kSelPer <= n) {
#pragma unroll
        for (int q = 0; q < kSelPer / 4; ++q) {
            const float4 f = *reinterpret_cast<const float4*>(vals + k0 + 4 * q);
            key[4 * q] = mag_bits(f.x);
            key[4 * q + 1] = mag_bits(f.y);
            key[4 * q + 2] = mag_bits(f.z);
            key[4 * q + 3] = mag_bits(f.w);
        }
    } else {
        // past the end: a key whose high bits never match the prefix
#pragma unroll
        for (int u = 0; u < kSelPer; ++u) key[u] = k0 + u < n ? mag_bits(vals[k0 + u]) : ~prefix;
    }
    uint32_t run_d = 0, run = 0;
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
        if (PASS > 0 && (key[u] & hi_mask) != (prefix & hi_mask)) continue;
        if (PASS == 0 && k0 + u >= n) continue;
        const uint32_t d = (key[u] >> shift) & 255u;
        if (d != run_d && run) {
            atomicAdd(&h[run_d], run);
            run = 0;
        }
        run_d = d;
        ++run;
    }
    if (run) atomicAdd(&h[run_d], run);
    __syncthreads();
    if (h[tid]) atomicAdd(&hist[PASS * kSelHist + (blockIdx.x % kSelCopies) * 256 + tid], h[tid]);
}

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// clear two bitmaps of `words` words (layers whose bitmap is large next to the entries)
__global__ void zero2_kernel(uint32_t* __restrict__ a, uint32_t* __restrict__ b, int64_t words)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x) {
        a[i] = 0u;
        b[i] = 0u;
    }
}

__device__ inline uint64_t cell_of(const int32_t* __restrict__ rows, const int32_t* __restrict__ cols, int64_t k,
                                   int32_t K)
{
    return (uint64_t)rows[k] * (uint64_t)K + (uint64_t)cols[k];
}

// Tiles of 4096 canonical entries (256 threads, four rounds of four entries).
constexpr int kKeepThreads = 256;
constexpr int kKeepTile = 4096;
constexpr int64_t kKeepDirect = 4096; // tiles whose tie prefix is summed directly

__device__ inline bool ties_partial(const uint32_t* __restrict__ state) { return state[1] + 1u != state[2]; }

__device__ inline int32_t block_excl(int32_t v, int32_t* smem /*[waves]*/, int32_t& total)
{
    constexpr int W = kKeepThreads / kWave;
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const int32_t inc = wave_incl(v);
    if (lane == kWave - 1) smem[w] = inc;
    __syncthreads();
    int32_t base = 0;
    total = 0;
#pragma unroll
    for (int i = 0; i < W; ++i) {
        const int32_t x = smem[i];
        if (i < w) base += x;
        total += x;
    }
    __syncthreads();
    return base + inc - v;
}

// Number of keys equal to T per tile; needed only when the ties are dropped in
// part (their rank in slot order then decides), otherwise the kernel returns.
__global__ void __launch_bounds__(kKeepThreads) eq_tiles_kernel(const int32_t* __restrict__ rows,
                                                                const int32_t* __restrict__ cols,
                                                                const float* __restrict__ vals, int64_t n, int32_t K,
                                                                uint32_t* __restrict__ state,
                                                                const uint32_t* __restrict__ hist,
                                                                int32_t* __restrict__ tile_eq,
                                                                uint32_t* __restrict__ kept_bm,
                                                                uint32_t* __restrict__ old_bm)
{
    __shared__ int32_t smem[kKeepThreads / kWave];
    // the word of this tile's first entry is the only one it may share with the
    // tile before, which both fill with atomic ORs: clear it for them
    if (threadIdx.x == 0 && blockIdx.x > 0) {
        const uint64_t w = cell_of(rows, cols, (int64_t)blockIdx.x * kKeepTile, K) >> 5;
        kept_bm[w] = 0u;
        old_bm[w] = 0u;
    }
    // the last pass's pick gives T, the rank among keys equal to T, and their count
    const SelPick pk = sel_pick(hist + (kSelPasses - 1) * kSelHist, state[3 + 3 * (kSelPasses - 2)],
                                state[4 + 3 * (kSelPasses - 2)], 0);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        state[0] = pk.prefix;
        state[1] = pk.rank;
        state[2] = pk.equal;
    }
    if (pk.rank + 1u == pk.equal) return;   // every key equal to T is dropped
    const uint32_t T = pk.prefix;
    const int64_t base = (int64_t)blockIdx.x * kKeepTile;
    int32_t c = 0;
    for (int i = threadIdx.x; i < kKeepTile; i += kKeepThreads) {
        const int64_t k = base + i;
        if (k < n && mag_bits(vals[k]) == T) ++c;
    }
    int32_t tot;
    block_excl(c, smem, tot);
    if (threadIdx.x == 0) tile_eq[blockIdx.x] = tot;
}

// The drop decision and the bitmaps, tile by tile.  An entry is dropped when
// its key is below T, or equal to T and among the first `ties` equal keys in
// slot order (the rank is counted only when ties are dropped in part).  The
// tile's cells ascend, so its bits fall in one contiguous run of bitmap words;
// the tile owns every word from its first entry's word up to the next tile's
// first entry's word (tile 0 also those before, the last tile those after) and
// stores each whole, zeros included, so the bitmaps need no clearing.  Only a
// tile's first and last words can hold another tile's bits: those two are
// combined with atomic ORs (the first word of every tile was cleared before).
// When the run fits in LDS the words are assembled there and stored coalesced;
// otherwise the tile clears the words it alone holds and every entry ORs its
// bits into global memory.  `old` gets every entry, `kept` the kept ones.  The
// values are copied for the rebuild.
constexpr int kKeepSpan = 4096;   // bitmap words assembled in LDS per tile

template <bool DIRECT>
__global__ void __launch_bounds__(kKeepThreads) keep_tiles_kernel(
    const int32_t* __restrict__ rows, const int32_t* __restrict__ cols, const float* __restrict__ vals, int64_t n,
    int32_t K, int64_t words, int cleared, const uint32_t* __restrict__ state, const int32_t* __restrict__ tile_eq,
    float* __restrict__ vcopy, uint32_t* __restrict__ kept_bm, uint32_t* __restrict__ old_bm)
{
    __shared__ uint32_t w_kept[kKeepSpan];
    __shared__ uint32_t w_old[kKeepSpan];
    __shared__ int32_t smem[kKeepThreads / kWave];
    __shared__ uint64_t s_first, s_last, s_end;
    __shared__ int s_pshared, s_nshared;
    const uint32_t T = state[0];
    const uint32_t ties = state[1] + 1u;
    const bool partial = ties_partial(state);
    const int64_t tile = blockIdx.x;
    const int64_t base = tile * kKeepTile;
    const int64_t cnt = n - base < kKeepTile ? n - base : kKeepTile;
    if (threadIdx.x == 0) {
        s_first = cell_of(rows, cols, base, K) >> 5;
        s_last = cell_of(rows, cols, base + cnt - 1, K) >> 5;
        // words up to (not including) the next tile's first word are this tile's
        const bool more = base + cnt < n;
        const uint64_t next = more ? cell_of(rows, cols, base + cnt, K) >> 5 : (uint64_t)words;
        s_end = next;
        s_nshared = more && next == s_last;
        s_pshared = tile > 0 && (cell_of(rows, cols, base - 1, K) >> 5) == s_first;
    }
    int32_t eqp = 0;
    if (partial) {
        if constexpr (DIRECT) {
            int32_t part = 0;
            for (int64_t i = threadIdx.x; i < tile; i += kKeepThreads) part += tile_eq[i];
            block_excl(part, smem, eqp);
        } else {
            eqp = tile_eq[tile];
        }
    }
    constexpr int R = kKeepTile / (kKeepThreads * 4);
    float v[R][4];
    int32_t r[R][4], c[R][4];
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const int64_t e0 = base + q * (kKeepThreads * 4) + 4 * threadIdx.x;
        if (e0 + 3 < n) {
            const float4 vv = *reinterpret_cast<const float4*>(vals + e0);
            const int4 rr = *reinterpret_cast<const int4*>(rows + e0);
            const int4 cc = *reinterpret_cast<const int4*>(cols + e0);
            v[q][0] = vv.x; v[q][1] = vv.y; v[q][2] = vv.z; v[q][3] = vv.w;
            r[q][0] = rr.x; r[q][1] = rr.y; r[q][2] = rr.z; r[q][3] = rr.w;
            c[q][0] = cc.x; c[q][1] = cc.y; c[q][2] = cc.z; c[q][3] = cc.w;
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const bool in = e0 + t < n;
                v[q][t] = in ? vals[e0 + t] : 0.0f;
                r[q][t] = in ? rows[e0 + t] : 0;
                c[q][t] = in ? cols[e0 + t] : 0;
            }
        }
    }
    __syncthreads();   // s_first, s_last, s_end, s_*shared
    const uint64_t wf = s_first, wl = s_last, we = s_end;
    const bool pshared = s_pshared != 0, nshared = s_nshared != 0;
    const bool in_lds = wl - wf < (uint64_t)kKeepSpan;
    // words this tile holds alone and no entry of it sets: before its first word
    // (tile 0) and between its last word and the next tile's first (a sparse
    // layer's bitmaps are cleared beforehand by a full grid instead)
    if (!cleared) {
        const uint64_t g0 = tile == 0 ? 0ull : wf;
        for (uint64_t w = g0 + threadIdx.x; w < wf; w += kKeepThreads) {
            kept_bm[w] = 0u;
            old_bm[w] = 0u;
        }
        for (uint64_t w = wl + 1 + threadIdx.x; w < we; w += kKeepThreads) {
            kept_bm[w] = 0u;
            old_bm[w] = 0u;
        }
    }
    if (in_lds) {
        for (int i = threadIdx.x; i <= (int)(wl - wf); i += kKeepThreads) {
            w_kept[i] = 0u;
            w_old[i] = 0u;
        }
    } else if (!cleared) {
        // the words of the run no other tile touches are cleared here first
        // (atomic stores: the ORs below are atomics on the same words)
        const int64_t c0 = (int64_t)wf + (pshared ? 1 : 0), c1 = (int64_t)wl - (nshared ? 1 : 0);
        for (int64_t w = c0 + threadIdx.x; w <= c1; w += kKeepThreads) {
            __hip_atomic_store(&kept_bm[w], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&old_bm[w], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __syncthreads();
    int32_t run = 0;   // equal keys of this tile in earlier rounds
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const int64_t e0 = base + q * (kKeepThreads * 4) + 4 * threadIdx.x;
        if (e0 + 3 < n) {
            *reinterpret_cast<float4*>(vcopy + e0) = make_float4(v[q][0], v[q][1], v[q][2], v[q][3]);
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (e0 + t < n) vcopy[e0 + t] = v[q][t];
        }
        uint32_t key[4];
        int32_t eq = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            key[t] = mag_bits(v[q][t]);
            eq += (e0 + t < n && key[t] == T) ? 1 : 0;
        }
        int32_t ex = 0, tot = 0;
        if (partial) ex = block_excl(eq, smem, tot);
        int32_t rank = eqp + run + ex;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (e0 + t >= n) continue;
            const bool keep = key[t] > T || (key[t] == T && partial && (uint32_t)rank >= ties);
            if (key[t] == T) ++rank;
            const uint64_t p = (uint64_t)r[q][t] * (uint64_t)K + (uint64_t)c[q][t];
            const uint32_t bit = 1u << (p & 31);
            if (in_lds) {
                const int i = (int)((p >> 5) - wf);
                atomicOr(&w_old[i], bit);
                if (keep) atomicOr(&w_kept[i], bit);
            } else {
                atomicOr(&old_bm[p >> 5], bit);
                if (keep) atomicOr(&kept_bm[p >> 5], bit);
            }
        }
        run += tot;
    }
    if (!in_lds) return;
    __syncthreads();
    const int span = (int)(wl - wf) + 1;
    for (int i = threadIdx.x; i < span; i += kKeepThreads) {
        const uint64_t w = wf + i;
        const uint32_t k = w_kept[i], o = w_old[i];
        if ((i == 0 && pshared) || (i == span - 1 && nshared)) {
            if (o) atomicOr(&old_bm[w], o);
            if (k) atomicOr(&kept_bm[w], k);
        } else {
            old_bm[w] = o;
            kept_bm[w] = k;
        }
    }
}

// ---- grow ------------------------------------------------------------------
// One batch takes the candidates t0 .. t0+T-1 in five launches, with no global
// atomic per candidate:
//   gen_bucket    every candidate's cell, grouped by region (2^rb consecutive
//                 cells, so a region owns whole bitmap words); a workgroup
//                 counts its candidates per region in LDS and reserves each
//                 region's run with one atomic.  The order inside a bucket is
//                 arbitrary: nothing downstream depends on it.
//   region_claim  one workgroup per region: the region's `occ` words in LDS,
//                 an LDS table keeps the smallest candidate index per free
//                 cell, the winners are marked accepted and their bits set,
//                 and the words are written back whole.
//   tile_sum/cut  accepted counts per tile of candidate indices; the tile
//                 holding the need-th accepted one is scanned to find it.
//   give_back     accepted candidates past that one clear their bits again.
// A region's bucket has a fixed capacity far above its expected size; if one
// ever overflows, the batch changes nothing and is taken again at half size
// (the outcome does not depend on the batch size).
constexpr int kGenThreads = 1024;
constexpr int kGenPer = 16;
constexpr int64_t kGenTile = (int64_t)kGenThreads * kGenPer;
constexpr int32_t kMaxRegions = 8192;
constexpr int kSubBits = 18;          // cells of one LDS pass of region_claim (a 32 KB bitmap)
constexpr int kClaimThreads = 1024;
constexpr int kTabBits = 13;
constexpr int kTabSlots = 1 << kTabBits;   // LDS table: 64 KB
constexpr int kTlBits = 21;           // candidate index within a batch
constexpr int64_t kSumTile = 8192;    // candidate indices per accepted-count tile
constexpr int kStOverflow = 12, kStTaken = 13, kStCut = 14;   // words of the prune state

static_assert(kMaxBatch <= (1ll << kTlBits), "candidate index must fit its field");
static_assert(kMaxBatch / kSumTile <= 1024, "one workgroup scans the tile counts");

__device__ inline uint64_t candidate_pos(uint64_t seed, uint64_t epoch, uint64_t t, uint64_t N)
{
    const uint64_t x = seed + ((epoch << 40) + t + 1ull) * kGamma;
    return __umul64hi(splitmix64_output(x), N);
}

__device__ inline uint32_t tab_slot(uint32_t c) { return (c * 0x9E3779B1u) >> (32 - kTabBits); }

// bucket entry: candidate index within the batch << 32 | cell within the region
__global__ void __launch_bounds__(kGenThreads) gen_bucket_kernel(uint64_t seed, uint64_t epoch, uint64_t t0,
                                                                 int64_t T, uint64_t N, int rb, int32_t R,
                                                                 int32_t cap, int32_t* __restrict__ fill,
                                                                 uint64_t* __restrict__ bucket,
                                                                 uint8_t* __restrict__ acc8,
                                                                 uint32_t* __restrict__ state)
{
    __shared__ int32_t cur[kMaxRegions];
    for (int32_t r = threadIdx.x; r < R; r += kGenThreads) cur[r] = 0;
    __syncthreads();
    const int64_t i0 = (int64_t)blockIdx.x * kGenTile + threadIdx.x;
    uint64_t pos[kGenPer];
#pragma unroll
    for (int u = 0; u < kGenPer; ++u) {
        const int64_t i = i0 + (int64_t)u * kGenThreads;
        pos[u] = candidate_pos(seed, epoch, t0 + (uint64_t)i, N);
        if (i < T) {
            atomicAdd(&cur[(int32_t)(pos[u] >> rb)], 1);
            acc8[i] = 0;
        }
    }
    __syncthreads();
    for (int32_t r = threadIdx.x; r < R; r += kGenThreads) {
        const int32_t c = cur[r];
        if (c) cur[r] = atomicAdd(&fill[r], c);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kGenPer; ++u) {
        const int64_t i = i0 + (int64_t)u * kGenThreads;
        if (i >= T) continue;
        const int32_t r = (int32_t)(pos[u] >> rb);
        const int32_t slot = atomicAdd(&cur[r], 1);
        if (slot < cap)
            bucket[(int64_t)r * cap + slot] = ((uint64_t)i << 32) | (uint64_t)(uint32_t)(pos[u] - ((uint64_t)r << rb));
        else
            atomicOr(&state[kStOverflow], 1u);
    }
}

// Region r in passes of 2^sb cells.  Table words pack cell << kTlBits | index,
// so an atomic minimum keeps the smallest index of a cell whatever the order.
// The table never fills: a pass holds at most 2^sb <= 4096 distinct cells when
// sb <= 12, and a bucket holds at most 4096 candidates otherwise.
__global__ void __launch_bounds__(kClaimThreads) region_claim_kernel(int rb, int sb, uint64_t words_total,
                                                                     int32_t cap, int32_t* __restrict__ fill,
                                                                     const uint64_t* __restrict__ bucket,
                                                                     const uint32_t* __restrict__ src_bm,
                                                                     uint32_t* __restrict__ occ_bm,
                                                                     uint8_t* __restrict__ acc8,
                                                                     const uint32_t* __restrict__ state)
{
    extern __shared__ unsigned long long tab[];   // kTabSlots words, then the pass's bitmap words
    uint32_t* bm = reinterpret_cast<uint32_t*>(tab + kTabSlots);
    __shared__ int32_t s_n, s_err;
    const int32_t r = blockIdx.x;
    if (threadIdx.x == 0) {
        const int32_t f = fill[r];
        s_n = f < cap ? f : cap;
        s_err = state[kStOverflow] != 0u;
        fill[r] = 0;   // ready for the next batch
    }
    __syncthreads();
    if (s_err) return;
    const int32_t n = s_n;
    const uint64_t* __restrict__ e = bucket + (int64_t)r * cap;
    const uint32_t cmask = (1u << sb) - 1u;
    const int passes = 1 << (rb - sb);
    for (int p = 0; p < passes; ++p) {
        const uint64_t w0 = (((uint64_t)r << rb) + ((uint64_t)p << sb)) >> 5;
        if (w0 >= words_total) break;   // uniform
        const uint64_t left = words_total - w0;
        const uint32_t nw = left < (uint64_t)(1u << (sb - 5)) ? (uint32_t)left : (1u << (sb - 5));
        for (uint32_t i = threadIdx.x; i < nw; i += kClaimThreads) bm[i] = src_bm[w0 + i];
        for (int i = threadIdx.x; i < kTabSlots; i += kClaimThreads) tab[i] = kEmpty;
        __syncthreads();
        for (int32_t k = threadIdx.x; k < n; k += kClaimThreads) {
            const uint64_t x = e[k];
            const uint32_t cell = (uint32_t)x;
            if ((cell >> sb) != (uint32_t)p) continue;
            const uint32_t c = cell & cmask;
            if ((bm[c >> 5] >> (c & 31)) & 1u) continue;
            const unsigned long long word = ((unsigned long long)c << kTlBits) | (x >> 32);
            uint32_t h = tab_slot(c);
            for (int probe = 0; probe < kTabSlots; ++probe) {
                const unsigned long long old = atomicCAS(&tab[h], (unsigned long long)kEmpty, word);
                if (old == kEmpty) break;
                if ((old >> kTlBits) == c) {
                    if (word < old) atomicMin(&tab[h], word);
                    break;
                }
                h = (h + 1u) & (kTabSlots - 1);
            }
        }
        __syncthreads();
        // a cell is in the table exactly when it was free; only now do bits change
        for (int32_t k = threadIdx.x; k < n; k += kClaimThreads) {
            const uint64_t x = e[k];
            const uint32_t cell = (uint32_t)x;
            if ((cell >> sb) != (uint32_t)p) continue;
            const uint32_t c = cell & cmask;
            const uint64_t tl = x >> 32;
            uint32_t h = tab_slot(c);
            for (int probe = 0; probe < kTabSlots; ++probe) {
                const unsigned long long w = tab[h];
                if (w == kEmpty) break;
                if ((w >> kTlBits) == c) {
                    if ((w & ((1ull << kTlBits) - 1ull)) == tl) {
                        acc8[tl] = 1;
                        atomicOr(&bm[c >> 5], 1u << (c & 31));
                    }
                    break;
                }
                h = (h + 1u) & (kTabSlots - 1);
            }
        }
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < nw; i += kClaimThreads) occ_bm[w0 + i] = bm[i];
        __syncthreads();
    }
}

// accepted candidates per tile of kSumTile indices (flags are 0/1 bytes)
__global__ void __launch_bounds__(256) tile_sum_kernel(const uint8_t* __restrict__ acc8, int64_t T,
                                                       int32_t* __restrict__ tsum, const uint32_t* __restrict__ state)
{
    __shared__ int32_t red[256 / kWave];
    if (state[kStOverflow]) return;
    const int64_t b0 = (int64_t)blockIdx.x * kSumTile;
    const int64_t b1 = b0 + kSumTile < T ? b0 + kSumTile : T;
    int32_t c = 0;
    for (int64_t i = b0 + 4 * threadIdx.x; i < b1; i += 4 * 256) {
        uint32_t w = *reinterpret_cast<const uint32_t*>(acc8 + i);
        if (i + 4 > b1) w &= (1u << (8 * (b1 - i))) - 1u;
        c += __popc(w);
    }
    c = wave_sum(c);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t t = 0;
        for (int i = 0; i < 256 / kWave; ++i) t += red[i];
        tsum[blockIdx.x] = t;
    }
}

// The first `need` accepted candidates in index order are taken, and the
// accepted ones at or past the cut give their cell back (few: the batch is
// sized to overshoot need only slightly).  Every workgroup finds the cut
// itself -- from the tile counts, then the flags of the tile where the
// running count reaches need -- so no launch of its own is spent on it.
// Workgroup 0 records how many were taken (state[kStTaken]; all when fewer
// than need were accepted) and writes the batch's result words (overflow,
// taken) to the host (`res`, mapped pinned memory, stored at system scope).
constexpr int kCutThreads = 256;
static_assert(kMaxBatch / kSumTile <= 4 * kCutThreads, "four tile counts per thread");
static_assert(kSumTile == 32 * kCutThreads, "32 flags of the cut tile per thread");

__device__ inline int32_t block_incl_256(int32_t v, int32_t* smem /*[4]*/)
{
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    int32_t inc = wave_incl(v);
    if (lane == kWave - 1) smem[w] = inc;
    __syncthreads();
    int32_t base = 0;
    for (int i = 0; i < w; ++i) base += smem[i];
    __syncthreads();
    return base + inc;
}

__global__ void __launch_bounds__(kCutThreads) cut_give_back_kernel(
    uint64_t seed, uint64_t epoch, uint64_t t0, int64_t T, uint64_t N, const int32_t* __restrict__ tsum,
    int32_t ntiles, int64_t need, const uint8_t* __restrict__ acc8, uint32_t* __restrict__ occ_bm,
    uint32_t* __restrict__ state, uint32_t* __restrict__ res)
{
    __shared__ int32_t smem[kCutThreads / kWave];
    __shared__ int32_t s_j, s_q, s_cut, s_all;
    const int tid = threadIdx.x;
    if (state[kStOverflow]) {
        if (blockIdx.x == 0 && tid == 0) {
            state[kStTaken] = 0u;
            __hip_atomic_store(&res[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            __hip_atomic_store(&res[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
        return;
    }
    // the tile where the running count first reaches need (four consecutive tiles per thread)
    int32_t v[4], loc = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int ti = 4 * tid + u;
        v[u] = ti < ntiles ? tsum[ti] : 0;
        loc += v[u];
    }
    const int32_t inc = block_incl_256(loc, smem);
    if (tid == 0) s_j = -1;
    if (tid == kCutThreads - 1) s_all = inc;
    __syncthreads();
    {
        int32_t run = inc - loc;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if ((int64_t)(run + v[u]) >= need && (int64_t)run < need) {
                s_j = 4 * tid + u;
                s_q = (int32_t)(need - run);
            }
            run += v[u];
        }
    }
    __syncthreads();
    const int32_t j = s_j;
    int64_t cut = T;
    uint32_t taken = (uint32_t)need;
    if (j < 0) {
        taken = (uint32_t)s_all;   // fewer than need accepted: all are taken
    } else {
        // the q-th accepted flag of tile j: 32 consecutive flags per thread
        const int32_t q = s_q;
        const int64_t lo = (int64_t)j * kSumTile + 32 * tid;
        uint8_t f[32];
        int32_t cnt = 0;
#pragma unroll
        for (int u = 0; u < 32; ++u) {
            f[u] = lo + u < T ? acc8[lo + u] : 0;
            cnt += f[u];
        }
        const int32_t ci = block_incl_256(cnt, smem);
        if (ci >= q && ci - cnt < q) {
            int32_t k = ci - cnt;
            for (int u = 0; u < 32; ++u) {
                k += f[u];
                if (f[u] && k == q) {
                    s_cut = (int32_t)(lo + u + 1);
                    break;
                }
            }
        }
        __syncthreads();
        cut = s_cut;
    }
    if (blockIdx.x == 0 && tid == 0) {
        state[kStTaken] = taken;
        state[kStCut] = (uint32_t)cut;
        __hip_atomic_store(&res[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __hip_atomic_store(&res[1], taken, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    for (int64_t i = cut + (int64_t)blockIdx.x * kCutThreads + tid; i < T; i += (int64_t)gridDim.x * kCutThreads) {
        if (!acc8[i]) continue;
        const uint64_t p = candidate_pos(seed, epoch, t0 + (uint64_t)i, N);
        atomicAnd(&occ_bm[p >> 5], ~(1u << (p & 31)));
    }
}

// Runs between a batch and a rebuild queued behind it before the host has
// seen the batch's result: when the batch overflowed or fell short, the old
// cells are put back into occ, so the rebuild sees a complete set of exactly
// nnz cells (its output is then replaced once the grow is redone).
struct GrowPlan {
    int rb, sb;
    int32_t R, cap;
};

// Regions hold about 2048 candidates (at most kMaxRegions regions); the bucket
// capacity is the mean plus eight standard deviations plus 64.
GrowPlan grow_plan(uint64_t N, int64_t T)
{
    GrowPlan g;
    int rb = 5;
    while (rb < kSubBits && ((uint64_t)T << (rb + 1)) <= 2048ull * N) ++rb;
    auto regions = [&](int b) { return (N + (1ull << b) - 1) >> b; };
    while (regions(rb) > (uint64_t)kMaxRegions) ++rb;
    g.rb = rb;
    g.sb = rb < kSubBits ? rb : kSubBits;
    g.R = (int32_t)regions(rb);
    const double mu = (double)T * (double)(1ull << rb) / (double)N;
    const double c = std::ceil(mu + 8.0 * std::sqrt(mu) + 64.0);
    g.cap = c >= (double)T ? (int32_t)T : (int32_t)c;
    return g;
}

// bucket entries any batch of at most `tmax` candidates can need: R * cap <=
// 2T + 8 sqrt(R * R mu) + 65 R with R mu <= 2T and R <= kMaxRegions
int64_t bucket_bound(uint64_t N, int64_t tmax)
{
    const double rmax = (double)std::min<uint64_t>((uint64_t)kMaxRegions, (N + 31) / 32);
    const double b = 2.0 * (double)tmax + 8.0 * std::sqrt(rmax * 2.0 * (double)tmax) + 65.0 * rmax + 1024.0;
    return (int64_t)std::ceil(b);
}

// ---- rebuild the canonical arrays from the bitmaps ---------------------------
// Units of 1024 bitmap words, one wavefront each (16 sweeps of one word per
// lane).  Kernel 1 counts each unit's bits in `occ` (the new entries) and in
// `old` (the entries before the drop).  Kernel 2 starts every unit at its
// prefix -- summed from the unit counts before it when there are few units,
// else read from their scans -- and, per sweep, turns the lanes' counts into
// slots with a wavefront scan: an occupied cell goes to the next slot; a kept
// cell takes the value the old entry at its old rank had.
constexpr int kEmitThreads = 256;
constexpr int kEmitSweeps = 8;
constexpr int64_t kEmitUnit = (int64_t)kWave * kEmitSweeps;   // words per wavefront
constexpr int64_t kEmitDirect = 16384;

__global__ void __launch_bounds__(kEmitThreads) bm_unit_counts_kernel(const uint32_t* __restrict__ occ_bm,
                                                                      const uint32_t* __restrict__ old_bm,
                                                                      int64_t words, int64_t units,
                                                                      int32_t* __restrict__ occ_cnt,
                                                                      int32_t* __restrict__ old_cnt)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t u = (int64_t)blockIdx.x * (kEmitThreads / kWave) + threadIdx.x / kWave;
    if (u >= units) return;
    int32_t a = 0, b = 0;
    for (int it = 0; it < kEmitSweeps; ++it) {
        const int64_t w = u * kEmitUnit + (int64_t)it * kWave + lane;
        if (w < words) {
            a += __popc(occ_bm[w]);
            b += __popc(old_bm[w]);
        }
    }
    a = wave_sum(a);
    b = wave_sum(b);
    if (lane == 0) {
        occ_cnt[u] = a;
        old_cnt[u] = b;
    }
}

// The bit walk is divergent (lanes hold different numbers of set bits), so it
// only records each entry -- row, column and the old slot its value comes from
// (-1: a grown cell, value 0) -- in a per-wave LDS list at the entry's offset
// from the list's first output slot; the list is then written out with every
// lane active, entries lane, lane+64, ..., so rows, cols and vals are stored as
// contiguous runs and the old values are read four at a time per lane.
constexpr int kEmitList = 512;   // entries per wave

__device__ inline void emit_flush(const int32_t* lr, const int32_t* lc, const int32_t* ls, int32_t n, int32_t out0,
                                  int32_t nnz, const float* __restrict__ vold, int32_t* __restrict__ rows,
                                  int32_t* __restrict__ cols, float* __restrict__ vals, uint16_t* __restrict__ cols16,
                                  int lane)
{
    if (n > nnz - out0) n = nnz - out0;   // never past the triple (occ holds nnz bits)
    __builtin_amdgcn_wave_barrier();
    for (int32_t i0 = 0; i0 < n; i0 += 4 * kWave) {
        float v[4];
        int32_t src[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int32_t i = i0 + q * kWave + lane;
            src[q] = i < n ? ls[i] : -1;
            v[q] = vold[src[q] >= 0 ? src[q] : 0];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int32_t i = i0 + q * kWave + lane;
            if (i < n) {
                rows[out0 + i] = lr[i];
                cols[out0 + i] = lc[i];
                if (cols16) cols16[out0 + i] = (uint16_t)lc[i];
                vals[out0 + i] = src[q] >= 0 ? v[q] : 0.0f;
            }
        }
    }
    __builtin_amdgcn_wave_barrier();
}

template <bool DIRECT, bool WIDE>
__global__ void __launch_bounds__(kEmitThreads) emit_units_kernel(
    const uint32_t* __restrict__ occ_bm, const uint32_t* __restrict__ kept_bm, const uint32_t* __restrict__ old_bm,
    int64_t words, int64_t units, const int32_t* __restrict__ occ_cnt, const int32_t* __restrict__ old_cnt,
    const float* __restrict__ vold, int64_t nnz, int32_t K, int32_t* __restrict__ rows, int32_t* __restrict__ cols,
    float* __restrict__ vals, uint16_t* __restrict__ cols16)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t u = (int64_t)blockIdx.x * (kEmitThreads / kWave) + threadIdx.x / kWave;
    // the workgroup's four units share one prefix: all threads sum the counts
    // of the units before the workgroup, each wave then adds its neighbours'
    __shared__ int32_t red[2][kEmitThreads / kWave];
    const int64_t u0 = (int64_t)blockIdx.x * (kEmitThreads / kWave);
    // slots fit 32 bits (nnz < 2^31)
    const int32_t nnz32 = (int32_t)nnz;
    int32_t run_o, run_d;
    if constexpr (DIRECT) {
        // eight loads of each count in flight per thread (clamped indexes, no branch around a load)
        int32_t a = 0, b = 0;
        for (int64_t i0 = threadIdx.x; i0 < u0; i0 += 8 * kEmitThreads) {
            int32_t x[8], y[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int64_t i = i0 + q * kEmitThreads;
                const int64_t ic = i < u0 ? i : 0;
                x[q] = occ_cnt[ic];
                y[q] = old_cnt[ic];
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const bool in = i0 + q * kEmitThreads < u0;
                a += in ? x[q] : 0;
                b += in ? y[q] : 0;
            }
        }
        a = wave_sum(a);
        b = wave_sum(b);
        if (lane == 0) {
            red[0][threadIdx.x / kWave] = a;
            red[1][threadIdx.x / kWave] = b;
        }
        __syncthreads();
        run_o = 0;
        run_d = 0;
        for (int i = 0; i < kEmitThreads / kWave; ++i) {
            run_o += red[0][i];
            run_d += red[1][i];
        }
        for (int64_t i = u0; i < u; ++i) {
            run_o += occ_cnt[i];
            run_d += old_cnt[i];
        }
    } else {
        run_o = u < units ? occ_cnt[u] : 0;
        run_d = u < units ? old_cnt[u] : 0;
    }
    __shared__ int32_t lr_[kEmitThreads / kWave][kEmitList];
    __shared__ int32_t lc_[kEmitThreads / kWave][kEmitList];
    __shared__ int32_t ls_[kEmitThreads / kWave][kEmitList];
    if (u >= units) return;
    int32_t* lr = lr_[threadIdx.x / kWave];
    int32_t* lc = lc_[threadIdx.x / kWave];
    int32_t* ls = ls_[threadIdx.x / kWave];
    int32_t nl = 0;      // entries in the list (wave-uniform)
    int32_t lout0 = 0;   // output slot of the list's first entry
    uint32_t om_[kEmitSweeps], dm_[kEmitSweeps], km_[kEmitSweeps];
#pragma unroll
    for (int it = 0; it < kEmitSweeps; ++it) {
        const int64_t w = u * kEmitUnit + (int64_t)it * kWave + lane;
        const bool in = w < words;
        om_[it] = in ? occ_bm[w] : 0u;
        dm_[it] = in ? old_bm[w] : 0u;
        km_[it] = in ? kept_bm[w] : 0u;
    }
#pragma unroll
    for (int it = 0; it < kEmitSweeps; ++it) {
        const int64_t w = u * kEmitUnit + (int64_t)it * kWave + lane;
        const uint32_t om = om_[it], dm = dm_[it], km = km_[it];
        const int32_t a = __popc(om), b = __popc(dm);
        const int32_t ia = wave_incl(a), ib = wave_incl(b);
        const int32_t ta = __builtin_amdgcn_readlane(ia, kWave - 1);
        const int32_t sweep0 = run_o;
        int32_t out = run_o + ia - a;
        const int32_t oldbase = run_d + ib - b;
        run_o += ta;
        run_d += __builtin_amdgcn_readlane(ib, kWave - 1);
        // the list takes this sweep if it fits (sweeps of a dense layer may not)
        const bool listed = ta <= kEmitList;
        if (nl > 0 && (!listed || nl + ta > kEmitList)) {
            emit_flush(lr, lc, ls, nl, lout0, nnz32, vold, rows, cols, vals, cols16, lane);
            nl = 0;
        }
        if (listed && nl == 0) lout0 = sweep0;
        int32_t lp = out - lout0;
        if (listed) nl += ta;
        if (!om) continue;
        int32_t r, c;
        if constexpr (WIDE) {
            const uint64_t p0 = (uint64_t)w << 5;
            const uint64_t rr = p0 / (uint64_t)K;
            r = (int32_t)rr;
            c = (int32_t)(p0 - rr * (uint64_t)K);
        } else {
            const uint32_t p0 = (uint32_t)w << 5;
            const uint32_t rr = p0 / (uint32_t)K;
            r = (int32_t)rr;
            c = (int32_t)(p0 - rr * (uint32_t)K);
        }
        int last = 0;
        uint32_t m = om;
        while (m && out < nnz32) {
            const int bit = __ffs(m) - 1;
            m &= m - 1u;
            c += bit - last;
            last = bit;
            while (c >= K) {
                c -= K;
                ++r;
            }
            const int32_t src = ((km >> bit) & 1u) ? oldbase + __popc(dm & ((1u << bit) - 1u)) : -1;
            if (listed) {
                lr[lp] = r;
                lc[lp] = c;
                ls[lp] = src;
                ++lp;
            } else {
                rows[out] = r;
                cols[out] = c;
                if (cols16) cols16[out] = (uint16_t)c;
                vals[out] = src >= 0 ? vold[src] : 0.0f;
            }
            ++out;
        }
    }
    if (nl > 0) emit_flush(lr, lc, ls, nl, lout0, nnz32, vold, rows, cols, vals, cols16, lane);
}

// ---- the column view from the new bitmap -----------------------------------
// The cells in tiles of 256 rows x 256 columns.  A tile's bits go to LDS row by
// row; ballots turn them into column words.  Pass 1 counts each column's entries
// per row block (and writes row_ptr from the word prefixes); after a scan of
// those counts down each column and across the column totals, pass 2 walks each
// column's bits in row order: an entry's transposed slot is its column's start
// in this row block plus its rank there, its canonical slot the word prefix of
// its row plus the bits before it.  A column's entries of one tile are written
// as one contiguous run, and the tiles of one column band are dispatched to one
// XCD, so the runs of neighbouring row blocks meet in the same L2.
constexpr int kCvDim = 256;              // rows and columns of a tile
constexpr int kCvWords = kCvDim / 32;    // bitmap words of a tile row
constexpr int kCvPad = kCvWords + 1;     // LDS row stride (spreads the banks)
constexpr int kCvThreads = 256;
constexpr int kXcds = 8;

struct CvTileShape {
    int32_t r0, c0, nrows, ncols;
};

__device__ inline CvTileShape cv_shape(int32_t bi, int32_t bj, int32_t M, int32_t K)
{
    CvTileShape t;
    t.r0 = bi * kCvDim;
    t.c0 = bj * kCvDim;
    t.nrows = M - t.r0 < kCvDim ? M - t.r0 : kCvDim;
    t.ncols = K - t.c0 < kCvDim ? K - t.c0 : kCvDim;
    return t;
}

// Tile of a workgroup: XCD x (workgroups are dealt to the XCDs in turn) owns
// the column bands [x * per, (x + 1) * per) and walks them row block by row
// block, so the bands that share bitmap lines, and the runs that neighbouring
// row blocks write into one column, meet in the same L2.  False past the grid.
__device__ inline bool cv_tile_of(int32_t nbi, int32_t nbj, int32_t& bi, int32_t& bj)
{
    const int32_t per = (nbj + kXcds - 1) / kXcds;
    const int32_t xcd = (int32_t)(blockIdx.x % kXcds), slot = (int32_t)(blockIdx.x / kXcds);
    bi = slot / per;
    bj = xcd * per + slot % per;
    return bi < nbi && bj < nbj;
}

// The tile's bits, row-major: rowbits[rr * kCvPad + i] holds columns
// c0+32i .. c0+32i+31 of tile row rr (zero outside the matrix).  Every thread
// issues all its loads (clamped indexes, both words of each unaligned span)
// before it writes any of them, so none waits behind another.
template <int T, int NB = 1>
__device__ inline void cv_load_rows(const uint32_t* const (&bm)[NB], uint64_t words, int32_t K, const CvTileShape& t,
                                    uint32_t* const (&rowbits)[NB])
{
    constexpr int R = kCvDim * kCvWords / T;
    uint32_t lo[NB][R], hi[NB][R];
    int sh[R];
#pragma unroll
    for (int n = 0; n < R; ++n) {
        const int q = threadIdx.x + n * T;
        const int rr = q / kCvWords, i = q % kCvWords;
        const bool in = rr < t.nrows && 32 * i < t.ncols;
        const uint64_t cell = in ? (uint64_t)(t.r0 + rr) * (uint64_t)K + (uint64_t)(t.c0 + 32 * i) : 0ull;
        const uint64_t w = cell >> 5, w1 = w + 1 < words ? w + 1 : w;
        sh[n] = (int)(cell & 31);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            lo[b][n] = bm[b][w];
            hi[b][n] = bm[b][w1];
        }
    }
#pragma unroll
    for (int n = 0; n < R; ++n) {
        const int q = threadIdx.x + n * T;
        const int rr = q / kCvWords, i = q % kCvWords;
        const int32_t valid = t.ncols - 32 * i;
        const uint32_t keep = valid >= 32 ? ~0u : (1u << (valid > 0 ? valid : 0)) - 1u;
        const bool live = rr < t.nrows && valid > 0;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const uint32_t x = sh[n] ? (lo[b][n] >> sh[n]) | (hi[b][n] << (32 - sh[n])) : lo[b][n];
            rowbits[b][rr * kCvPad + i] = live ? (x & keep) : 0u;
        }
    }
}

template <int T>
__device__ inline void cv_load_rows(const uint32_t* bm, uint64_t words, int32_t K, const CvTileShape& t,
                                    uint32_t* rowbits)
{
    const uint32_t* const src[1] = {bm};
    uint32_t* const dst[1] = {rowbits};
    cv_load_rows<T, 1>(src, words, K, t, dst);
}

// Column words: colbits[c * kCvPad + j] holds rows 32j .. 32j+31 of column c.
// The tile is 8 x 8 blocks of 32 x 32 bits; a block sits in 32 lanes (lane l
// holds row l) and five butterfly stages exchange ever smaller sub-blocks
// with the lane 16, 8, 4, 2, 1 away, after which lane l holds column l.
template <int T>
__device__ inline void cv_transpose(const uint32_t* rowbits, uint32_t* colbits)
{
    const int lane = threadIdx.x & (kWave - 1), l = lane & 31;
    for (int blk = 2 * (int)(threadIdx.x / kWave) + (lane >> 5); blk < kCvWords * kCvWords; blk += T / 32) {
        const int j = blk / kCvWords, i = blk % kCvWords;
        uint32_t x = rowbits[(32 * j + l) * kCvPad + i];
#pragma unroll
        for (int st = 0; st < 5; ++st) {
            const int d = 16 >> st;
            const uint32_t m = st == 0 ? 0x0000FFFFu : st == 1 ? 0x00FF00FFu : st == 2 ? 0x0F0F0F0Fu
                             : st == 3 ? 0x33333333u : 0x55555555u;
            const uint32_t y = __shfl_xor(x, d, kWave);
            x = (l & d) ? (((y >> d) & m) | (x & ~m)) : ((x & m) | ((y << d) & ~m));
        }
        colbits[(32 * i + l) * kCvPad + j] = x;
    }
}

// ---- count and scan passes of the rebuild ---------------------------------
// Pass 1 (one workgroup per tile): each column's entries in the tile (cnt,
// [row block][K]), and each row's entries in the tile, new and old (rcnt and
// ocnt, [column block][M]).  With `guard` (a rebuild queued behind a grow batch
// before its result is known): when that batch did not complete the grow
// (overflow, or fewer than `need` taken), occ is first put back to the cells
// before the drop, so that it holds exactly nnz cells and the rebuild stays
// inside the arrays; the grow is then taken again and the layer rebuilt once
// more.
__global__ void __launch_bounds__(kCvThreads) cv_count_kernel(
    uint32_t* __restrict__ occ_bm, const uint32_t* __restrict__ old_bm, uint64_t words, int32_t M, int32_t K,
    int32_t nbi, int32_t nbj, int64_t nnz, int32_t* __restrict__ cnt, int32_t* __restrict__ rcnt,
    int32_t* __restrict__ ocnt, int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_ptr,
    int32_t* __restrict__ n_empty_r, int32_t* __restrict__ n_empty_c, const uint32_t* __restrict__ guard,
    uint32_t need)
{
    __shared__ uint32_t rowbits[kCvDim * kCvPad];
    __shared__ uint32_t colbits[kCvDim * kCvPad];
    __shared__ uint32_t oldbits[kCvDim * kCvPad];
    const bool restore = guard && !(guard[kStOverflow] == 0u && guard[kStTaken] == need);
    if (restore) {   // every workgroup reads the old cells below, so the copy races with no read
        const int64_t step = (int64_t)gridDim.x * kCvThreads;
        for (int64_t w = (int64_t)blockIdx.x * kCvThreads + threadIdx.x; w < (int64_t)words; w += step)
            occ_bm[w] = old_bm[w];
    }
    int32_t bi, bj;
    if (!cv_tile_of(nbi, nbj, bi, bj)) return;
    const CvTileShape t = cv_shape(bi, bj, M, K);
    const int tid = threadIdx.x;
    if (bi == 0 && bj == 0 && tid == 0) {
        row_ptr[M] = (int32_t)nnz;
        col_ptr[K] = (int32_t)nnz;
        *n_empty_r = 0;   // the views' empty-key lists are rebuilt at the end
        *n_empty_c = 0;
    }
    {
        const uint32_t* const src[2] = {restore ? old_bm : occ_bm, old_bm};
        uint32_t* const dst[2] = {rowbits, oldbits};
        cv_load_rows<kCvThreads, 2>(src, words, K, t, dst);
    }
    __syncthreads();
    {
        int32_t rc = 0, oc = 0;
#pragma unroll
        for (int i = 0; i < kCvWords; ++i) {
            rc += __popc(rowbits[tid * kCvPad + i]);
            oc += __popc(oldbits[tid * kCvPad + i]);
        }
        if (tid < t.nrows) {
            rcnt[(int64_t)bj * M + t.r0 + tid] = rc;
            ocnt[(int64_t)bj * M + t.r0 + tid] = oc;
        }
    }
    cv_transpose<kCvThreads>(rowbits, colbits);
    __syncthreads();
    int32_t c = 0;
#pragma unroll
    for (int j = 0; j < kCvWords; ++j) c += __popc(colbits[tid * kCvPad + j]);
    if (tid < t.ncols) cnt[(int64_t)bi * K + t.c0 + tid] = c;
}

// counts a[0], a[stride], ... (n of them) -> their exclusive prefix, in place; returns the total
__device__ inline int32_t cv_scan_down(int32_t* __restrict__ a, int64_t stride, int32_t n)
{
    constexpr int kBatch = 16;   // loads in flight per thread
    int32_t run = 0;
    for (int32_t b0 = 0; b0 < n; b0 += kBatch) {
        int32_t v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) v[u] = b0 + u < n ? a[(int64_t)(b0 + u) * stride] : 0;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (b0 + u < n) a[(int64_t)(b0 + u) * stride] = run;
            run += v[u];
        }
    }
    return run;
}

// a workgroup's sum of one value per thread (kCvDim threads)
__device__ inline int32_t cv_block_sum(int32_t v, int32_t* red /*[kCvDim / kWave]*/)
{
    const int32_t ws = wave_sum(v);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = ws;
    __syncthreads();
    int32_t t = 0;
    for (int i = 0; i < kCvDim / kWave; ++i) t += red[i];
    return t;
}

// Pass 2: workgroups [0, nbj) take a band of kCvDim columns each: the counts
// down each column become prefixes over the row blocks, the column totals and
// the band's sum go out.  Workgroups [nbj, nbj + nbi) do the same for a band of
// kCvDim rows, across the column blocks, for the new and the old cells.
__global__ void __launch_bounds__(kCvDim) cv_scan_kernel(int32_t* __restrict__ cnt, int32_t* __restrict__ rcnt,
                                                         int32_t* __restrict__ ocnt, int32_t nbi, int32_t nbj,
                                                         int32_t M, int32_t K, int32_t* __restrict__ tot,
                                                         int32_t* __restrict__ band, int32_t* __restrict__ rtot,
                                                         int32_t* __restrict__ rband, int32_t* __restrict__ otot,
                                                         int32_t* __restrict__ oband)
{
    __shared__ int32_t red[kCvDim / kWave];
    if ((int32_t)blockIdx.x < nbj) {
        const int64_t c = (int64_t)blockIdx.x * kCvDim + threadIdx.x;
        int32_t run = 0;
        if (c < K) {
            run = cv_scan_down(cnt + c, K, nbi);
            tot[c] = run;
        }
        const int32_t s = cv_block_sum(run, red);
        if (threadIdx.x == 0) band[blockIdx.x] = s;
        return;
    }
    const int32_t b = (int32_t)blockIdx.x - nbj;
    const int64_t r = (int64_t)b * kCvDim + threadIdx.x;
    int32_t rn = 0, ro = 0;
    if (r < M) {
        rn = cv_scan_down(rcnt + r, M, nbj);
        ro = cv_scan_down(ocnt + r, M, nbj);
        rtot[r] = rn;
        otot[r] = ro;
    }
    const int32_t sn = cv_block_sum(rn, red);
    __syncthreads();
    const int32_t so = cv_block_sum(ro, red);
    if (threadIdx.x == 0) {
        rband[b] = sn;
        oband[b] = so;
    }
}

// last index i in [0, n) with a[i] <= x (a ascending, a[0] <= x)
__device__ inline int32_t cv_last_le(const int32_t* a, int32_t n, int32_t x)
{
    int32_t lo = 0, hi = n;
    while (hi - lo > 1) {
        const int32_t mid = (lo + hi) >> 1;
        if (a[mid] <= x) lo = mid;
        else hi = mid;
    }
    return lo;
}

// The slice tables of both views (null where a width has none): row view
// (keys rows, slices over columns) and column view (keys columns, slices over rows).
struct CvTabs {
    int32_t rS[kTileWidths], cS[kTileWidths];
    int32_t* rtab[kTileWidths];
    int32_t* ctab[kTileWidths];
};

// The slice boundaries that fall inside one tile, per side (0: the row
// view's, along the columns; 1: the column view's, along the rows) and batch
// width: s = lo .. lo + n - 1, boundary s at tile offset off[s] (the last tile
// along a side also takes s = S, whose offset is the side's length).  One
// thread per (side, width, s) computes its boundary once.
struct CvBounds {
    int32_t lo[2][kTileWidths], n[2][kTileWidths];
    int16_t off[2][kTileWidths][kMaxSplits + 1];
};

__device__ inline void cv_bounds_init(CvBounds& cb)
{
    if (threadIdx.x < 2 * kTileWidths) {
        (&cb.lo[0][0])[threadIdx.x] = kMaxSplits + 1;
        (&cb.n[0][0])[threadIdx.x] = 0;
    }
}

__device__ inline void cv_bounds_find(CvBounds& cb, const CvTabs& tabs, const CvTileShape& t, int32_t M, int32_t K,
                                      bool last_r, bool last_c)
{
    constexpr int PER = kMaxSplits + 1;
    const int q = (int)threadIdx.x;
    if (q >= 2 * kTileWidths * PER) return;
    const int side = q / (kTileWidths * PER), w = (q / PER) % kTileWidths, s = q % PER;
    const int32_t S = side == 0 ? tabs.rS[w] : tabs.cS[w];
    const bool has = side == 0 ? tabs.rtab[w] != nullptr : tabs.ctab[w] != nullptr;
    if (!has || s > S) return;
    const int32_t nidx = side == 0 ? K : M;
    const int32_t o0 = side == 0 ? t.c0 : t.r0, len = side == 0 ? t.ncols : t.nrows;
    const bool last = side == 0 ? last_r : last_c;
    const int32_t b = split_start(s, S, nidx);
    if ((b >= o0 && b < o0 + len) || (s == S && last)) {
        cb.off[side][w][s] = (int16_t)(b - o0);
        atomicMin(&cb.lo[side][w], s);
        atomicAdd(&cb.n[side][w], 1);
    }
}

// a view's slice-table entries at one side's boundaries inside the tile, for
// key a (< nkey) along the other side: slot of the key's first entry in the
// tile (`first`) plus its entries before the boundary (word prefixes `pre` and
// the bits of the boundary's word)
__device__ inline void cv_tab_side(int32_t* tab, const CvBounds& cb, int side, int w, int32_t nkeys, int32_t key0,
                                   int a, int32_t nkey, int32_t first, const uint8_t* pre, const uint32_t* bits,
                                   int32_t total)
{
    const int32_t lo = cb.lo[side][w], n = cb.n[side][w];
    if (a >= nkey) return;
    for (int32_t s = lo; s < lo + n; ++s) {
        const int32_t lb = cb.off[side][w][s];
        const int32_t before = lb >= kCvDim ? total
                               : pre[a * kCvWords + (lb >> 5)] + __popc(bits[a * kCvPad + (lb >> 5)] & ((1u << (lb & 31)) - 1u));
        tab[(int64_t)s * nkeys + key0 + a] = first + before;
    }
}

constexpr int kCvScatterThreads = 1024;
constexpr int32_t kCvStage = 4096;   // tile entries handled through LDS lists

// Pass 3, one tile per workgroup: both index views and the canonical triple.
// Entries are numbered twice inside the tile: x in row order (a row's entries
// are consecutive canonical slots, starting at rowk) and e in column order (a
// column's entries are consecutive transposed slots, starting at colbase).  A
// walk over each row word's bits lists the row and column of every x; a pass
// in x order (striped across the threads) finds each entry's e from the
// column words and, for a kept cell, its old slot from the old cells' words,
// reads its value from the copy taken before the drop (a grown cell is +0),
// writes the canonical triple and iperm as row runs and leaves value, row and
// column at e in LDS, from where a pass in e order writes rows_t and vals_t as
// column runs.  A tile with more than kCvStage entries finds each entry's
// column by binary search and reads and writes global memory directly.
struct CvScatterOut {
    int32_t* row_ptr;
    int32_t* col_ptr;
    int32_t* rows;
    int32_t* cols;
    float* vals;
    uint16_t* cols16;   // or null
    int32_t* rows_t;
    float* vals_t;
    int32_t* iperm;
    uint16_t* rows_t16;   // or null
};

// a band scan's start for the thread's key (one of kCvDim, in waves 4q .. 4q+3
// of the workgroup): the bands before this one, plus the exclusive prefix of
// the band's totals; `tot_here` is the thread's own total (0 past the matrix)
struct CvBandScan {
    int32_t incl, own, boff;
};

__device__ inline CvBandScan cv_band_scan_a(const int32_t* __restrict__ band, int32_t nb_before, int32_t tot_here,
                                            int32_t* wsum /*[kCvDim / kWave]*/)
{
    const int lane = threadIdx.x & (kWave - 1);
    CvBandScan b;
    b.own = tot_here;
    int32_t o = 0;
    for (int32_t i = lane; i < nb_before; i += kWave) o += band[i];
    b.boff = wave_sum(o);
    b.incl = wave_incl(tot_here);
    if (lane == kWave - 1) wsum[(threadIdx.x / kWave) % (kCvDim / kWave)] = b.incl;
    return b;
}

__device__ inline int32_t cv_band_scan_b(const CvBandScan& b, const int32_t* wsum)
{
    int32_t start = b.boff + b.incl - b.own;
    const int w = (threadIdx.x / kWave) % (kCvDim / kWave);
    for (int i = 0; i < w; ++i) start += wsum[i];
    return start;
}

__global__ void __launch_bounds__(kCvScatterThreads) cv_scatter_kernel(
    const uint32_t* __restrict__ occ_bm, const uint32_t* __restrict__ old_bm, const uint32_t* __restrict__ kept_bm,
    uint64_t words, int32_t M, int32_t K, int32_t nbi, int32_t nbj, const int32_t* __restrict__ cnt,
    const int32_t* __restrict__ tot, const int32_t* __restrict__ band, const int32_t* __restrict__ rcnt,
    const int32_t* __restrict__ rtot, const int32_t* __restrict__ rband, const int32_t* __restrict__ ocnt,
    const int32_t* __restrict__ otot, const int32_t* __restrict__ oband, const float* __restrict__ vcopy,
    CvScatterOut out, CvTabs tabs)
{
    __shared__ uint32_t rowbits[kCvDim * kCvPad];    // rows of the new cells; later erow, ecol
    __shared__ uint32_t colbits[kCvDim * kCvPad];
    __shared__ uint32_t oldbits[kCvDim * kCvPad];
    __shared__ uint32_t keptbits[kCvDim * kCvPad];
    __shared__ uint8_t rwp[kCvDim * kCvWords];    // entries of a row before each of its words
    __shared__ uint8_t cwp[kCvDim * kCvWords];    // entries of a column before each of its words
    __shared__ uint8_t owp[kCvDim * kCvWords];    // old cells of a row before each of its words
    __shared__ int32_t rowk[kCvDim];              // canonical slot of a row's first entry in the tile
    __shared__ int32_t orowk[kCvDim];             // old slot of a row's first old cell in the tile
    __shared__ int32_t rowoff[kCvDim + 1];        // x of a row's first entry
    __shared__ int32_t colstart[kCvDim + 1];      // e of a column's first entry
    __shared__ int32_t colbase[kCvDim];           // transposed slot of a column's first entry
    __shared__ uint8_t xrow[kCvStage];   // row of x
    __shared__ uint8_t xcol[kCvStage];   // column of x
    __shared__ float sval[kCvStage];     // value of e
    __shared__ int32_t red[2][kCvDim / kWave];
    __shared__ int32_t wsum[3][kCvDim / kWave];
    __shared__ CvBounds cb;
    static_assert(2 * kCvStage <= (int)sizeof(rowbits), "erow and ecol fit the new cells' rows");
    uint8_t* erow = reinterpret_cast<uint8_t*>(rowbits);   // row of e (x pass on)
    uint8_t* ecol = erow + kCvStage;                        // column of e
    int32_t bi, bj;
    if (!cv_tile_of(nbi, nbj, bi, bj)) return;
    const CvTileShape t = cv_shape(bi, bj, M, K);
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;

    cv_bounds_init(cb);
    {
        const uint32_t* const src[3] = {occ_bm, old_bm, kept_bm};
        uint32_t* const dst[3] = {rowbits, oldbits, keptbits};
        cv_load_rows<kCvScatterThreads, 3>(src, words, K, t, dst);
    }
    // first slots: waves 0-3 the columns' transposed ones (column starts also to col_ptr from the
    // first row block), 4-7 the rows' canonical ones (row starts to row_ptr from the first column
    // block), 8-11 the rows' old ones: the bands before this one, a scan of the band's totals, and
    // the key's entries in the blocks before this tile
    const int role = wv / (kCvDim / kWave);   // uniform per wave
    const int a = tid % kCvDim;
    CvBandScan bs{0, 0, 0};
    int32_t before_tile = 0;
    if (role == 0) {
        const int32_t c = t.c0 + (a < t.ncols ? a : t.ncols - 1);
        before_tile = cnt[(int64_t)bi * K + c];
        bs = cv_band_scan_a(band, bj, a < t.ncols ? tot[c] : 0, wsum[0]);
    } else if (role == 1 || role == 2) {
        const int32_t r = t.r0 + (a < t.nrows ? a : t.nrows - 1);
        const bool nw = role == 1;
        before_tile = (nw ? rcnt : ocnt)[(int64_t)bj * M + r];
        bs = cv_band_scan_a(nw ? rband : oband, bi, a < t.nrows ? (nw ? rtot : otot)[r] : 0, wsum[role]);
    }
    __syncthreads();
    if (role == 0) {
        const int32_t start = cv_band_scan_b(bs, wsum[0]);
        colbase[a] = a < t.ncols ? start + before_tile : 0;
        if (bi == 0 && a < t.ncols) out.col_ptr[t.c0 + a] = start;
    } else if (role == 1) {
        const int32_t start = cv_band_scan_b(bs, wsum[1]);
        rowk[a] = a < t.nrows ? start + before_tile : 0;
        if (bj == 0 && a < t.nrows) out.row_ptr[t.r0 + a] = start;
    } else if (role == 2) {
        const int32_t start = cv_band_scan_b(bs, wsum[2]);
        orowk[a] = a < t.nrows ? start + before_tile : 0;
    }
    cv_transpose<kCvScatterThreads>(rowbits, colbits);
    cv_bounds_find(cb, tabs, t, M, K, bj == nbj - 1, bi == nbi - 1);
    __syncthreads();
    // word prefixes and counts: threads 0..255 rows, 256..511 columns, 512..767 the old cells' rows
    int32_t cntv = 0;
    if (tid < 3 * kCvDim) {
        const uint32_t* bits = role == 0 ? rowbits : role == 1 ? colbits : oldbits;
        uint8_t* pre = role == 0 ? rwp : role == 1 ? cwp : owp;
#pragma unroll
        for (int i = 0; i < kCvWords; ++i) {
            pre[a * kCvWords + i] = (uint8_t)cntv;
            cntv += __popc(bits[a * kCvPad + i]);
        }
        if (role < 2) {
            const int32_t inc = wave_incl(cntv);
            if (lane == kWave - 1) red[role][a / kWave] = inc;
        }
    }
    __syncthreads();
    if (tid < 2 * kCvDim) {
        const bool row = role == 0;
        int32_t before = 0;
        for (int i = 0; i < a / kWave; ++i) before += red[role][i];
        const int32_t ex = before + wave_incl(cntv) - cntv;
        (row ? rowoff : colstart)[a] = ex;
        if (a == kCvDim - 1) (row ? rowoff : colstart)[kCvDim] = ex + cntv;
    }
    __syncthreads();
    // slice tables: threads 0..255 the rows' entries (row view), 256..511 the columns'
    if (tid < 2 * kCvDim) {
        const bool row = role == 0;
        for (int w = 0; w < kTileWidths; ++w) {
            if (row && tabs.rtab[w]) {
                const int32_t total = a < t.nrows ? rowoff[a + 1] - rowoff[a] : 0;
                cv_tab_side(tabs.rtab[w], cb, 0, w, M, t.r0, a, t.nrows, a < t.nrows ? rowk[a] : 0, rwp, rowbits,
                            total);
            }
            if (!row && tabs.ctab[w]) {
                const int32_t total = a < t.ncols ? colstart[a + 1] - colstart[a] : 0;
                cv_tab_side(tabs.ctab[w], cb, 1, w, K, t.c0, a, t.ncols, a < t.ncols ? colbase[a] : 0, cwp, colbits,
                            total);
            }
        }
    }
    const int32_t E = colstart[kCvDim];
    // a kept cell's value from the copy taken before the drop (its old slot: the row's first old
    // cell in the tile plus the old cells before it); a grown cell is +0
    auto old_slot = [&](int rr, int c) -> int32_t {
        const int ci = c >> 5;
        const uint32_t below = (1u << (c & 31)) - 1u;
        if (!((keptbits[rr * kCvPad + ci] >> (c & 31)) & 1u)) return -1;
        return orowk[rr] + owp[rr * kCvWords + ci] + __popc(oldbits[rr * kCvPad + ci] & below);
    };
    if (E <= kCvStage) {   // uniform
        // row and column of every x: two row words per thread
#pragma unroll
        for (int n = 0; n < kCvDim * kCvWords / kCvScatterThreads; ++n) {
            const int q = tid + n * kCvScatterThreads;
            const int ra = q / kCvWords, i = q % kCvWords;
            uint32_t m = rowbits[ra * kCvPad + i];
            int32_t x = rowoff[ra] + rwp[ra * kCvWords + i];
            while (m) {
                xrow[x] = (uint8_t)ra;
                xcol[x] = (uint8_t)(32 * i + __ffs(m) - 1);
                m &= m - 1u;
                ++x;
            }
        }
        __syncthreads();   // rowbits is dead from here: erow and ecol take its place
        {
            // x order: the old values read (all R loads in flight first), the canonical triple and
            // iperm written, (value, row, column) to e
            constexpr int R = kCvStage / kCvScatterThreads;
            float v[R];
            int32_t src[R];
#pragma unroll
            for (int u = 0; u < R; ++u) {
                const int32_t x = tid + u * kCvScatterThreads;
                src[u] = x < E ? old_slot(xrow[x], xcol[x]) : -1;
                v[u] = vcopy[src[u] >= 0 ? src[u] : 0];
            }
#pragma unroll
            for (int u = 0; u < R; ++u) {
                const int32_t x = tid + u * kCvScatterThreads;
                if (x < E) {
                    const int rr = xrow[x], c = xcol[x];
                    const float val = src[u] >= 0 ? v[u] : 0.0f;
                    const int32_t k = rowk[rr] + (x - rowoff[rr]);
                    const int j = rr >> 5;
                    const int32_t before =
                        cwp[c * kCvWords + j] + __popc(colbits[c * kCvPad + j] & ((1u << (rr & 31)) - 1u));
                    const int32_t e = colstart[c] + before;
                    out.rows[k] = t.r0 + rr;
                    out.cols[k] = t.c0 + c;
                    if (out.cols16) out.cols16[k] = (uint16_t)(t.c0 + c);
                    out.vals[k] = val;
                    out.iperm[k] = colbase[c] + before;
                    sval[e] = val;
                    erow[e] = (uint8_t)rr;
                    ecol[e] = (uint8_t)c;
                }
            }
        }
        __syncthreads();
        // e order: the column runs of rows_t and vals_t
        for (int32_t e = tid; e < E; e += kCvScatterThreads) {
            const int c = ecol[e];
            const int32_t kt = colbase[c] + (e - colstart[c]);
            const int32_t r = t.r0 + erow[e];
            out.rows_t[kt] = r;
            if (out.rows_t16) out.rows_t16[kt] = (uint16_t)r;
            out.vals_t[kt] = sval[e];
        }
        return;
    }
    // a dense tile: column by binary search, row by a walk of the column's words
    for (int32_t e = tid; e < E; e += kCvScatterThreads) {
        const int32_t c = cv_last_le(colstart, kCvDim, e);
        int32_t rank = e - colstart[c];
        const int32_t kt = colbase[c] + rank;
        int j = 0;
        uint32_t m = colbits[c * kCvPad];
        for (int n = __popc(m); rank >= n; n = __popc(m)) {
            rank -= n;
            m = colbits[c * kCvPad + (++j)];
        }
        for (; rank > 0; --rank) m &= m - 1u;
        const int rr = 32 * j + __ffs(m) - 1;
        const int ci = c >> 5;
        const int32_t k = rowk[rr] + rwp[rr * kCvWords + ci] + __popc(rowbits[rr * kCvPad + ci] & ((1u << (c & 31)) - 1u));
        const int32_t src = old_slot(rr, c);
        const float val = src >= 0 ? vcopy[src] : 0.0f;
        out.rows[k] = t.r0 + rr;
        out.cols[k] = t.c0 + c;
        if (out.cols16) out.cols16[k] = (uint16_t)(t.c0 + c);
        out.vals[k] = val;
        out.rows_t[kt] = t.r0 + rr;
        if (out.rows_t16) out.rows_t16[kt] = (uint16_t)(t.r0 + rr);
        out.vals_t[kt] = val;
        out.iperm[k] = kt;
    }
}

struct PruneScratch {
    uint32_t* state;    // [16]
    uint32_t* hist;     // [kSelPasses * kSelHist] selection histograms
    int32_t* tile_eq;   // [keep tiles] keys equal to T per tile (then their scan)
    float* vcopy;       // [nnz] the values before the rebuild
    uint32_t* kept_bm;  // [words]
    uint32_t* occ_bm;   // [words]
    uint32_t* old_bm;   // [words] cells of the entries before the drop
    int32_t* occ_cnt;   // [units] occupied bits per emit unit (then their scan)
    int32_t* old_cnt;   // [units] old bits per emit unit
    uint8_t* acc8;      // [tmax] accepted flag per candidate of the batch
    int32_t* tsum;      // [tmax / kSumTile] accepted per tile
    int32_t* fill;      // [kMaxRegions] bucket fill per region
    uint64_t* bucket;   // [nbucket] candidates grouped by region
    int32_t* cvcnt;     // [row blocks * K] entries per column and row block, then their prefixes
    int32_t* cvtot;     // [K] entries per column
    int32_t* cvband;    // [column blocks] entries per band of kCvDim columns
    int32_t* rcnt;      // [column blocks * M] entries per row and column block, then their prefixes
    int32_t* ocnt;      // [column blocks * M] the same for the cells before the drop
    int32_t* rtot;      // [M] entries per row
    int32_t* otot;      // [M] cells before the drop per row
    int32_t* rband;     // [row blocks] entries per band of kCvDim rows
    int32_t* oband;     // [row blocks] cells before the drop per band of rows
    uint32_t* gstate;   // [16] gradient grow: thresholds and counts
    uint32_t* ghist;    // [kGradHistWords] gradient grow: digit histograms
    int32_t* tie_cnt;   // [M * grad_col_tiles(K)] gradient grow: threshold ties per row and column tile
    void* scan;         // scan scratch
    int64_t tmax, words, units, ktiles, nbucket;
};

// The column view is rebuilt from the bitmap when the bitmap is small next to
// the entries (two passes over it cost less than sorting the entries);
// otherwise by the general index build.
inline bool cv_from_bitmap(const snack_layer* L)
{
    const uint64_t N = (uint64_t)L->M * (uint64_t)L->K;
    return L->nnz > 0 && N <= 256ull * (uint64_t)L->nnz;
}

int64_t batch_cap(const snack_layer* L)
{
    int64_t t = L->nnz + 4096;
    if (t < 65536) t = 65536;
    if (t > kMaxBatch) t = kMaxBatch;
    return t;
}

size_t layout(const snack_layer* L, PruneScratch* ps)
{
    const int64_t n = L->nnz > 0 ? L->nnz : 1;
    const uint64_t N = (uint64_t)L->M * (uint64_t)L->K;
    const int64_t words = (int64_t)((N + 31) / 32);
    const int64_t units = (words + kEmitUnit - 1) / kEmitUnit;
    const int64_t ktiles = (n + kKeepTile - 1) / kKeepTile;
    const int64_t tm = batch_cap(L);
    const int64_t nb = bucket_bound(N, tm);
    const int64_t nbi = (L->M + kCvDim - 1) / kCvDim;
    int64_t sn = units > ktiles ? units : ktiles;
    if (L->K > sn) sn = L->K;
    const int64_t nties = (int64_t)L->M * grad_col_tiles(L->K);
    if (nties > sn) sn = nties;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += al(bytes);
        return o;
    };
    size_t o_state = take(16 * 4), o_hist = take((size_t)kSelPasses * kSelHist * 4);
    size_t o_teq = take((size_t)ktiles * 4), o_vc = take((size_t)n * 4);
    size_t o_kbm = take((size_t)words * 4), o_obm = take((size_t)words * 4), o_dbm = take((size_t)words * 4);
    size_t o_oc = take((size_t)units * 4), o_dc = take((size_t)units * 4);
    size_t o_acc = take((size_t)tm + 8), o_tsum = take((size_t)(tm / kSumTile + 1) * 4);
    size_t o_fill = take((size_t)kMaxRegions * 4), o_bucket = take((size_t)nb * 8);
    const int64_t nbj = (L->K + kCvDim - 1) / kCvDim;
    size_t o_cvcnt = take((size_t)nbi * L->K * 4), o_cvtot = take((size_t)L->K * 4);
    size_t o_cvband = take((size_t)nbj * 4);
    size_t o_rcnt = take((size_t)nbj * L->M * 4), o_ocnt = take((size_t)nbj * L->M * 4);
    size_t o_rtot = take((size_t)L->M * 4), o_otot = take((size_t)L->M * 4);
    size_t o_rband = take((size_t)nbi * 4), o_oband = take((size_t)nbi * 4);
    size_t o_gst = take(16 * 4), o_gh = take((size_t)kGradHistWords * 4), o_tie = take((size_t)nties * 4);
    size_t o_scan = take(scan_scratch_bytes(sn));
    if (ps) {
        char* base = (char*)L->scratch;
        ps->state = (uint32_t*)(base + o_state);
        ps->hist = (uint32_t*)(base + o_hist);
        ps->tile_eq = (int32_t*)(base + o_teq);
        ps->vcopy = (float*)(base + o_vc);
        ps->kept_bm = (uint32_t*)(base + o_kbm);
        ps->occ_bm = (uint32_t*)(base + o_obm);
        ps->old_bm = (uint32_t*)(base + o_dbm);
        ps->occ_cnt = (int32_t*)(base + o_oc);
        ps->old_cnt = (int32_t*)(base + o_dc);
        ps->acc8 = (uint8_t*)(base + o_acc);
        ps->tsum = (int32_t*)(base + o_tsum);
        ps->fill = (int32_t*)(base + o_fill);
        ps->bucket = (uint64_t*)(base + o_bucket);
        ps->cvcnt = (int32_t*)(base + o_cvcnt);
        ps->cvtot = (int32_t*)(base + o_cvtot);
        ps->cvband = (int32_t*)(base + o_cvband);
        ps->rcnt = (int32_t*)(base + o_rcnt);
        ps->ocnt = (int32_t*)(base + o_ocnt);
        ps->rtot = (int32_t*)(base + o_rtot);
        ps->otot = (int32_t*)(base + o_otot);
        ps->rband = (int32_t*)(base + o_rband);
        ps->oband = (int32_t*)(base + o_oband);
        ps->gstate = (uint32_t*)(base + o_gst);
        ps->ghist = (uint32_t*)(base + o_gh);
        ps->tie_cnt = (int32_t*)(base + o_tie);
        ps->scan = base + o_scan;
        ps->tmax = tm;
        ps->words = words;
        ps->units = units;
        ps->ktiles = ktiles;
        ps->nbucket = nb;
    }
    return off + 256;
}

}  // namespace

size_t prune_scratch_bytes(const snack_layer* L)
{
    const uint64_t N = (uint64_t)L->M * (uint64_t)L->K;
    if (N > kMaxBitmapBits) return 0;
    return layout(L, nullptr);
}

namespace {

// The canonical arrays and both views from the occupancy bitmap.
snack_status rebuild(snack_layer* L, const PruneScratch& ps, hipStream_t s, const uint32_t* guard = nullptr,
                     uint32_t need = 0)
{
    const int64_t nnz = L->nnz;
    const uint64_t N = (uint64_t)L->M * (uint64_t)L->K;
    if (cv_from_bitmap(L)) {
        // count, scan, then one pass over the tiles writes the canonical triple (with its 16-bit
        // column copy), the column view (with its 16-bit row copy) and the slice tables
        ProfScope pc(KC_CANON, s);
        const int32_t M = L->M, K = L->K;
        const int32_t nbi = (M + kCvDim - 1) / kCvDim, nbj = (K + kCvDim - 1) / kCvDim;
        const uint64_t words = (uint64_t)ps.words;
        const int64_t nslots = (int64_t)kXcds * ((nbj + kXcds - 1) / kXcds) * nbi;
        hipLaunchKernelGGL(cv_count_kernel, dim3((unsigned)nslots), dim3(kCvThreads), 0, s, ps.occ_bm, ps.old_bm, words,
                           M, K, nbi, nbj, nnz, ps.cvcnt, ps.rcnt, ps.ocnt, L->row_ptr, L->col_ptr, L->fwd.n_empty,
                           L->tr.n_empty, guard, need);
        hipLaunchKernelGGL(cv_scan_kernel, dim3((unsigned)(nbj + nbi)), dim3(kCvDim), 0, s, ps.cvcnt, ps.rcnt, ps.ocnt,
                           nbi, nbj, M, K, ps.cvtot, ps.cvband, ps.rtot, ps.rband, ps.otot, ps.oband);
        SNACK_HIP(hipGetLastError());
        CvTabs tabs;
        for (int w = 0; w < kTileWidths; ++w) {
            tabs.rS[w] = L->fwd.split[w].S;
            tabs.rtab[w] = L->fwd.split[w].S >= 2 ? L->fwd.split[w].tab : nullptr;
            tabs.cS[w] = L->tr.split[w].S;
            tabs.ctab[w] = L->tr.split[w].S >= 2 ? L->tr.split[w].tab : nullptr;
        }
        CvScatterOut o;
        o.row_ptr = L->row_ptr;
        o.col_ptr = L->col_ptr;
        o.rows = L->rows;
        o.cols = L->cols;
        o.vals = L->vals;
        o.cols16 = L->fwd.idx16;
        o.rows_t = L->rows_t;
        o.vals_t = L->vals_t;
        o.iperm = L->iperm;
        o.rows_t16 = L->tr.idx16;
        hipLaunchKernelGGL(cv_scatter_kernel, dim3((unsigned)nslots), dim3(kCvScatterThreads), 0, s, ps.occ_bm,
                           ps.old_bm, ps.kept_bm, words, M, K, nbi, nbj, ps.cvcnt, ps.cvtot, ps.cvband, ps.rcnt,
                           ps.rtot, ps.rband, ps.ocnt, ps.otot, ps.oband, ps.vcopy, o, tabs);
        SNACK_HIP(hipGetLastError());
        SNACK_CHECK(canon_index_tail(L, s, /*idx16_done=*/true, /*empty_cleared=*/true));
        for (int w = 0; w < kTileWidths; ++w) {
            if (tabs.rtab[w]) L->fwd.split[w].valid = true;
            if (tabs.ctab[w]) L->tr.split[w].valid = true;
        }
        return SNACK_OK;
    }
    // ---- a layer too sparse for the tiles: the canonical arrays from the bitmap in unit order,
    // then the index build ----
    if (guard) return SNACK_ERR_INVALID_ARG;   // only the tile rebuild is queued ahead of a grow result
    const int64_t nu = ps.units;
    const unsigned grid = (unsigned)((nu + (kEmitThreads / kWave) - 1) / (kEmitThreads / kWave));
    hipLaunchKernelGGL(bm_unit_counts_kernel, dim3(grid), dim3(kEmitThreads), 0, s, ps.occ_bm, ps.old_bm, ps.words,
                       nu, ps.occ_cnt, ps.old_cnt);
    SNACK_HIP(hipGetLastError());
    const bool direct = nu <= kEmitDirect;
    if (!direct) {
        SNACK_CHECK(exclusive_scan_i32(ps.occ_cnt, ps.occ_cnt, nu, nullptr, ps.scan, s));
        SNACK_CHECK(exclusive_scan_i32(ps.old_cnt, ps.old_cnt, nu, nullptr, ps.scan, s));
    }
    const bool wide = N > 0xFFFFFFFFull;
    auto emit = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(kEmitThreads), 0, s, ps.occ_bm, ps.kept_bm, ps.old_bm, ps.words,
                           nu, ps.occ_cnt, ps.old_cnt, ps.vcopy, nnz, L->K, L->rows, L->cols, L->vals,
                           (uint16_t*)nullptr);
    };
    if (direct) {
        if (wide) emit(emit_units_kernel<true, true>);
        else emit(emit_units_kernel<true, false>);
    } else {
        if (wide) emit(emit_units_kernel<false, true>);
        else emit(emit_units_kernel<false, false>);
    }
    SNACK_HIP(hipGetLastError());
    return canon_build_index(L, s);
}

}  // namespace

// The drop: the n_drop smallest magnitudes (order key: IEEE bits of |v|, then
// slot) leave; kept_bm holds the kept cells, old_bm every cell before the
// drop, vcopy the values.
snack_status drop_stage(snack_layer* L, const PruneScratch& ps, int64_t n_drop, hipStream_t s)
{
    const int64_t nnz = L->nnz;
    // ---- drop: the n_drop-th smallest magnitude key T and its tie rank ----
    {
        hipLaunchKernelGGL(prune_init_kernel, dim3(32), dim3(256), 0, s, ps.state, ps.hist, (uint32_t)(n_drop - 1),
                           ps.fill, kMaxRegions);
        const unsigned nsel = (unsigned)((nnz + (int64_t)kSelThreads * kSelPer - 1) / ((int64_t)kSelThreads * kSelPer));
        hipLaunchKernelGGL(sel_pass_kernel<0>, dim3(nsel), dim3(kSelThreads), 0, s, L->vals, nnz, ps.state, ps.hist);
        hipLaunchKernelGGL(sel_pass_kernel<1>, dim3(nsel), dim3(kSelThreads), 0, s, L->vals, nnz, ps.state, ps.hist);
        hipLaunchKernelGGL(sel_pass_kernel<2>, dim3(nsel), dim3(kSelThreads), 0, s, L->vals, nnz, ps.state, ps.hist);
        hipLaunchKernelGGL(sel_pass_kernel<3>, dim3(nsel), dim3(kSelThreads), 0, s, L->vals, nnz, ps.state, ps.hist);
        SNACK_HIP(hipGetLastError());
        hipLaunchKernelGGL(eq_tiles_kernel, dim3((unsigned)ps.ktiles), dim3(kKeepThreads), 0, s, L->rows, L->cols,
                           L->vals, nnz, L->K, ps.state, ps.hist, ps.tile_eq, ps.kept_bm, ps.old_bm);
        // a sparse layer's bitmap is cleared by a full grid (the tiles would each clear long gaps)
        const int cleared = ps.words > ps.ktiles * (int64_t)kKeepSpan ? 1 : 0;
        if (cleared)
            hipLaunchKernelGGL(zero2_kernel, dim3(grid_for(ps.words)), dim3(kThreads), 0, s, ps.kept_bm, ps.old_bm,
                               ps.words);
        SNACK_HIP(hipGetLastError());
        if (ps.ktiles <= kKeepDirect) {
            hipLaunchKernelGGL(keep_tiles_kernel<true>, dim3((unsigned)ps.ktiles), dim3(kKeepThreads), 0, s, L->rows,
                               L->cols, L->vals, nnz, L->K, ps.words, cleared, ps.state, ps.tile_eq, ps.vcopy, ps.kept_bm,
                               ps.old_bm);
        } else {
            // a scan of zeros when every tie is dropped (the counts were not written then; they are not used)
            SNACK_CHECK(exclusive_scan_i32(ps.tile_eq, ps.tile_eq, ps.ktiles, nullptr, ps.scan, s));
            hipLaunchKernelGGL(keep_tiles_kernel<false>, dim3((unsigned)ps.ktiles), dim3(kKeepThreads), 0, s, L->rows,
                               L->cols, L->vals, nnz, L->K, ps.words, cleared, ps.state, ps.tile_eq, ps.vcopy, ps.kept_bm,
                               ps.old_bm);
        }
        SNACK_HIP(hipGetLastError());
    }
    return SNACK_OK;
}

snack_status prune_regrow(snack_layer* L, int64_t n_drop, hipStream_t s)
{
    const int64_t nnz = L->nnz;
    const uint64_t N = (uint64_t)L->M * (uint64_t)L->K;
    if (n_drop == 0) {
        L->epoch += 1;
        return SNACK_OK;
    }
    if (N > kMaxBitmapBits || L->scratch_bytes < layout(L, nullptr)) return SNACK_ERR_UNSUPPORTED;
    ProfScope prof(KC_PRUNE, s);
    PruneScratch ps;
    layout(L, &ps);
    const int64_t kept = nnz - n_drop;
    SNACK_CHECK(drop_stage(L, ps, n_drop, s));

    // ---- grow: walk the candidate stream in batches ----
    int64_t need = n_drop;
    int64_t got = 0;
    uint64_t t0 = 0;
    int batches = 0;
    int shrink = 0;   // halvings of the batch after a bucket overflow
    bool claimed = false;   // a batch has written occ
    const uint64_t words_total = (uint64_t)ps.words;
    // The first batch nearly always completes the grow, so the rebuild is
    // queued right behind it, before its result is read (the host would
    // otherwise leave the GPU idle while it waits and relaunches); its first
    // kernel keeps that rebuild consistent if the batch did not complete it,
    // and the grow then starts over from the kept cells.  Only the bitmap
    // rebuild qualifies: it uses no scratch that the grow needs.
    bool speculate = cv_from_bitmap(L);
    bool rebuilt = false;
    while (need > 0) {
        const double p_empty = (double)(N - (uint64_t)kept - (uint64_t)got) / (double)N;
        double want = (double)need / (p_empty > 1e-9 ? p_empty : 1e-9) * 1.03 + 4096.0;
        int64_t T = want > (double)ps.tmax ? ps.tmax : (int64_t)want;
        T >>= shrink;
        if (T < 1) T = 1;
        GrowPlan g = grow_plan(N, T);
        if (L->grow_cap_max > 0 && g.cap > L->grow_cap_max) g.cap = L->grow_cap_max;
        const size_t lds = (size_t)kTabSlots * 8 + ((size_t)1 << g.sb) / 8;
        if ((int64_t)g.R * g.cap > ps.nbucket || lds > (size_t)L->lds_bytes) return SNACK_ERR_UNSUPPORTED;
        const unsigned ntiles = (unsigned)((T + kGenTile - 1) / kGenTile);
        const int32_t nsum = (int32_t)((T + kSumTile - 1) / kSumTile);
        hipLaunchKernelGGL(gen_bucket_kernel, dim3(ntiles), dim3(kGenThreads), 0, s, L->seed, L->epoch, t0, T, N,
                           g.rb, g.R, g.cap, ps.fill, ps.bucket, ps.acc8, ps.state);
        // the first batch starts from the kept cells (occ is first written, whole, by this pass)
        hipLaunchKernelGGL(region_claim_kernel, dim3((unsigned)g.R), dim3(kClaimThreads), lds, s, g.rb, g.sb,
                           words_total, g.cap, ps.fill, ps.bucket, claimed ? ps.occ_bm : ps.kept_bm, ps.occ_bm,
                           ps.acc8, ps.state);
        hipLaunchKernelGGL(tile_sum_kernel, dim3((unsigned)nsum), dim3(256), 0, s, ps.acc8, T, ps.tsum, ps.state);
        // the cut, the give-back and the result words (overflow, taken) written to the host
        hipLaunchKernelGGL(cut_give_back_kernel, dim3(grid_for(T) < 256u ? grid_for(T) : 256u), dim3(kCutThreads), 0,
                           s, L->seed, L->epoch, t0, T, N, ps.tsum, nsum, need, ps.acc8, ps.occ_bm, ps.state,
                           L->host_res_dev);
        SNACK_HIP(hipGetLastError());
        SNACK_HIP(hipEventRecord(L->grow_ev, s));
        const bool queued = speculate;
        if (queued) {
            SNACK_CHECK(rebuild(L, ps, s, ps.state, (uint32_t)need));
            speculate = false;
        }
        SNACK_HIP(hipEventSynchronize(L->grow_ev));
        const volatile uint32_t* hr = L->host_res;
        const uint32_t res[2] = {hr[0], hr[1]};
        if (++batches > 100000) return SNACK_ERR_UNSUPPORTED;
        if (queued) {
            if (res[0] == 0u && (int64_t)res[1] == need) {
                rebuilt = true;
                break;
            }
            // the guard has put the old cells back: take the grow again from the start
            if (res[0]) {
                hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(kThreads), 0, s, ps.state + kStOverflow,
                                   (int64_t)1, 0u);
                SNACK_HIP(hipGetLastError());
                ++shrink;
            }
            need = n_drop;
            got = 0;
            t0 = 0;
            claimed = false;
            continue;
        }
        if (res[0]) {   // nothing was changed: take the same candidates in a smaller batch
            hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(kThreads), 0, s, ps.state + kStOverflow, (int64_t)1, 0u);
            SNACK_HIP(hipGetLastError());
            ++shrink;
            continue;
        }
        shrink = 0;
        claimed = true;
        const int64_t taken = (int64_t)res[1];
        got += taken;
        need -= taken;
        t0 += (uint64_t)T;
    }

    if (!rebuilt) SNACK_CHECK(rebuild(L, ps, s));
    L->epoch += 1;
    return SNACK_OK;
}

// Row-local: each row drops and regrows inside itself (rows.hip writes the
// bitmaps), then the same rebuild.
snack_status prune_regrow_rows(snack_layer* L, int64_t num, int64_t den, bool gradient, const float* X,
                               const float* dY, int32_t B, hipStream_t s)
{
    const uint64_t N = (uint64_t)L->M * (uint64_t)L->K;
    if (num == 0 || L->nnz == 0) {
        L->epoch += 1;
        return SNACK_OK;
    }
    if (N > kMaxBitmapBits || L->scratch_bytes < layout(L, nullptr)) return SNACK_ERR_UNSUPPORTED;
    if (rows_lds_per_wave(L->K) > L->lds_bytes) return SNACK_ERR_UNSUPPORTED;
    ProfScope prof(KC_PRUNE, s);
    PruneScratch ps;
    layout(L, &ps);
    RowDst r;
    r.row_ptr = L->row_ptr;
    r.cols = L->cols;
    r.vals = L->vals;
    r.vcopy = ps.vcopy;
    r.old_bm = ps.old_bm;
    r.kept_bm = ps.kept_bm;
    r.occ_bm = ps.occ_bm;
    r.M = L->M;
    r.K = L->K;
    r.num = num;
    r.den = den;
    r.gradient = gradient;
    r.seed = L->seed;
    r.epoch = L->epoch;
    r.X = X;
    r.dY = dY;
    r.B = B;
    SNACK_CHECK(rows_drop_grow(r, L->lds_bytes, s));
    SNACK_CHECK(rebuild(L, ps, s));
    L->epoch += 1;
    return SNACK_OK;
}

snack_status prune_regrow_grad(snack_layer* L, int64_t n_drop, const float* X, const float* dY, int32_t B,
                               hipStream_t s)
{
    const uint64_t N = (uint64_t)L->M * (uint64_t)L->K;
    if (n_drop == 0) {
        L->epoch += 1;
        return SNACK_OK;
    }
    if (N >= (1ull << 32) || L->scratch_bytes < layout(L, nullptr)) return SNACK_ERR_UNSUPPORTED;
    ProfScope prof(KC_PRUNE, s);
    PruneScratch ps;
    layout(L, &ps);
    SNACK_CHECK(drop_stage(L, ps, n_drop, s));
    GradGrow g;
    g.kept_bm = ps.kept_bm;
    g.occ_bm = ps.occ_bm;
    g.words = ps.words;
    g.need = n_drop;
    g.X = X;
    g.dY = dY;
    g.B = B;
    g.state = ps.gstate;
    g.hist = ps.ghist;
    g.tie_cnt = ps.tie_cnt;
    g.scan = ps.scan;
    SNACK_CHECK(grow_by_gradient(L, g, s));
    SNACK_CHECK(rebuild(L, ps, s));
    L->epoch += 1;
    return SNACK_OK;
}

}  // namespace snack
