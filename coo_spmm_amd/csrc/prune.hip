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
#include "internal.h"

namespace snack {
namespace {

constexpr int kThreads = 256;
constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr int64_t kMaxBatch = 1 << 21;          // candidates per batch
constexpr int kTBits = 21;                       // candidate index bits in a table word
constexpr int kHashBits = 22;                    // table slots (load <= 1/2)
constexpr uint64_t kEmpty = ~0ull;
constexpr uint64_t kMaxBitmapBits = 1ull << 34;
constexpr int kSelBlocks = 512;                  // workgroups of one selection pass

static_assert(kMaxBatch <= (1ll << kTBits), "candidate index must fit its field");

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

// ---- drop: radix select ---------------------------------------------------
// state: [0] prefix, [1] rank still to find among keys matching the prefix,
// [2] number of keys equal to the final prefix (set by the last pass).
// A thread adds runs of equal digits before touching LDS, which keeps the
// first passes (where nearly every key shares a digit) free of contention;
// each workgroup then adds its nonzero bins to the global histogram.
__global__ void __launch_bounds__(kThreads) sel_hist_kernel(const float* __restrict__ vals, int64_t n,
                                                            const uint32_t* __restrict__ state, int shift,
                                                            uint32_t* __restrict__ hist)
{
    __shared__ uint32_t h[256];
    h[threadIdx.x] = 0;
    __syncthreads();
    const uint32_t prefix = state[0];
    const uint32_t hi_mask = (shift >= 24) ? 0u : (0xFFFFFFFFu << (shift + 8));
    uint32_t run_d = 0, run = 0;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t key = mag_bits(vals[k]);
        if ((key & hi_mask) != (prefix & hi_mask)) continue;
        const uint32_t d = (key >> shift) & 255u;
        if (d != run_d && run) {
            atomicAdd(&h[run_d], run);
            run = 0;
        }
        run_d = d;
        ++run;
    }
    if (run) atomicAdd(&h[run_d], run);
    __syncthreads();
    if (h[threadIdx.x]) atomicAdd(&hist[threadIdx.x], h[threadIdx.x]);
}

// picks the digit holding the wanted rank, then clears the histogram for the next pass
__global__ void __launch_bounds__(256) sel_pick_kernel(uint32_t* __restrict__ hist, uint32_t* __restrict__ state,
                                                       int shift)
{
    __shared__ uint32_t tot[256];
    tot[threadIdx.x] = hist[threadIdx.x];
    __syncthreads();
    hist[threadIdx.x] = 0;
    if (threadIdx.x == 0) {
        uint32_t r = state[1];
        uint32_t dg = 0;
        for (; dg < 255; ++dg) {
            if (r < tot[dg]) break;
            r -= tot[dg];
        }
        state[0] |= dg << shift;
        state[1] = r;
        if (shift == 0) state[2] = tot[dg];
    }
}

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// zero four bitmaps of `words` words in one launch
__global__ void zero4_kernel(uint32_t* __restrict__ a, uint32_t* __restrict__ b, uint32_t* __restrict__ c,
                             uint32_t* __restrict__ d, int64_t words)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x) {
        a[i] = 0u;
        b[i] = 0u;
        c[i] = 0u;
        d[i] = 0u;
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
    int32_t inc = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int32_t o = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += o;
    }
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
__global__ void __launch_bounds__(kKeepThreads) eq_tiles_kernel(const float* __restrict__ vals, int64_t n,
                                                                const uint32_t* __restrict__ state,
                                                                int32_t* __restrict__ tile_eq)
{
    __shared__ int32_t smem[kKeepThreads / kWave];
    if (!ties_partial(state)) return;
    const uint32_t T = state[0];
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
// tile's cells ascend, so its bits fall in one contiguous run of bitmap words:
// when the run fits in LDS the words are assembled there and stored coalesced
// (the first and last word, which neighbouring tiles may share, with atomic
// ORs); otherwise every entry ORs its bits into global memory.  `old` gets
// every entry, `kept` and `occ` the kept ones (bitmaps zero beforehand).  The
// values are copied for the rebuild.
constexpr int kKeepSpan = 4096;   // bitmap words assembled in LDS per tile

template <bool DIRECT>
__global__ void __launch_bounds__(kKeepThreads) keep_tiles_kernel(
    const int32_t* __restrict__ rows, const int32_t* __restrict__ cols, const float* __restrict__ vals, int64_t n,
    int32_t K, const uint32_t* __restrict__ state, const int32_t* __restrict__ tile_eq, float* __restrict__ vcopy,
    uint32_t* __restrict__ kept_bm, uint32_t* __restrict__ occ_bm, uint32_t* __restrict__ old_bm)
{
    __shared__ uint32_t w_kept[kKeepSpan];
    __shared__ uint32_t w_old[kKeepSpan];
    __shared__ int32_t smem[kKeepThreads / kWave];
    __shared__ uint64_t s_first, s_last;
    const uint32_t T = state[0];
    const uint32_t ties = state[1] + 1u;
    const bool partial = ties_partial(state);
    const int64_t tile = blockIdx.x;
    const int64_t base = tile * kKeepTile;
    const int64_t cnt = n - base < kKeepTile ? n - base : kKeepTile;
    if (threadIdx.x == 0) {
        s_first = cell_of(rows, cols, base, K) >> 5;
        s_last = cell_of(rows, cols, base + cnt - 1, K) >> 5;
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
    __syncthreads();   // s_first, s_last
    const uint64_t wf = s_first, wl = s_last;
    const bool in_lds = wl - wf < (uint64_t)kKeepSpan;
    if (in_lds) {
        for (int i = threadIdx.x; i <= (int)(wl - wf); i += kKeepThreads) {
            w_kept[i] = 0u;
            w_old[i] = 0u;
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
                if (keep) {
                    atomicOr(&kept_bm[p >> 5], bit);
                    atomicOr(&occ_bm[p >> 5], bit);
                }
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
        if (i == 0 || i == span - 1) {
            if (o) atomicOr(&old_bm[w], o);
            if (k) {
                atomicOr(&kept_bm[w], k);
                atomicOr(&occ_bm[w], k);
            }
        } else {
            old_bm[w] = o;
            kept_bm[w] = k;
            occ_bm[w] = k;
        }
    }
}

// ---- grow ------------------------------------------------------------------
// candidate i of this batch is stream element t0 + i; occupied cells get the sentinel N
__global__ void gen_candidates_kernel(uint64_t seed, uint64_t epoch, uint64_t t0, int64_t T, uint64_t N,
                                      const uint32_t* __restrict__ occ_bm, uint64_t* __restrict__ cpos)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < T; i += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t t = t0 + (uint64_t)i;
        const uint64_t x = seed + ((epoch << 40) + t + 1ull) * kGamma;
        const uint64_t pos = __umul64hi(splitmix64_output(x), N);
        const bool occupied = (occ_bm[pos >> 5] >> (pos & 31)) & 1u;
        cpos[i] = occupied ? N : pos;
    }
}

__global__ void hash_clear_kernel(unsigned long long* __restrict__ tab, int64_t H)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < H; i += (int64_t)gridDim.x * blockDim.x)
        tab[i] = kEmpty;
}

__device__ inline uint32_t hash_slot(uint64_t pos) { return (uint32_t)((pos * kGamma) >> (64 - kHashBits)); }

// Every free candidate claims its cell in `occ`.  Occupied cells were filtered
// out when the batch was generated, so a claim that finds its bit already set
// lost to another candidate of this batch: the cell is marked contested.
__global__ void claim_kernel(const uint64_t* __restrict__ cpos, int64_t T, uint64_t N, uint32_t* __restrict__ occ_bm,
                             uint32_t* __restrict__ con_bm)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < T; i += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t p = cpos[i];
        if (p >= N) continue;
        const uint32_t bit = 1u << (p & 31);
        const uint32_t old = atomicOr(&occ_bm[p >> 5], bit);
        if (old & bit) atomicOr(&con_bm[p >> 5], bit);
    }
}

// Claimants of contested cells register (cell, index) in an open-addressing
// table; the word packs cell << kTBits | index, so an atomic minimum keeps the
// smallest index whatever the order of the atomics.
__global__ void contest_kernel(const uint64_t* __restrict__ cpos, int64_t T, uint64_t N,
                               const uint32_t* __restrict__ con_bm, unsigned long long* __restrict__ tab,
                               int32_t* __restrict__ cflag)
{
    const uint32_t mask = (1u << kHashBits) - 1u;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < T; i += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t p = cpos[i];
        int32_t f = 0;
        if (p < N && ((con_bm[p >> 5] >> (p & 31)) & 1u)) {
            f = 1;
            const unsigned long long word = (p << kTBits) | (uint64_t)i;
            uint32_t h = hash_slot(p);
            for (uint32_t probe = 0; probe <= mask; ++probe) {
                const unsigned long long old = atomicCAS(&tab[h], (unsigned long long)kEmpty, word);
                if (old == kEmpty) break;
                if ((old >> kTBits) == p) {
                    if (word < old) atomicMin(&tab[h], word);
                    break;
                }
                h = (h + 1u) & mask;
            }
        }
        cflag[i] = f;
    }
}

// accepted[i] = candidate i is free and the first (smallest index) to name its cell
__global__ void accept_kernel(const uint64_t* __restrict__ cpos, int64_t T, uint64_t N,
                              const int32_t* __restrict__ cflag, const unsigned long long* __restrict__ tab,
                              int32_t* __restrict__ accepted)
{
    const uint32_t mask = (1u << kHashBits) - 1u;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < T; i += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t p = cpos[i];
        int32_t a = 0;
        if (p < N) {
            if (!cflag[i]) {
                a = 1;
            } else {
                uint32_t h = hash_slot(p);
                for (uint32_t probe = 0; probe <= mask; ++probe) {
                    const unsigned long long w = tab[h];
                    if (w == kEmpty) break;
                    if ((w >> kTBits) == p) {
                        a = (w & ((1ull << kTBits) - 1ull)) == (uint64_t)i ? 1 : 0;
                        break;
                    }
                    h = (h + 1u) & mask;
                }
            }
        }
        accepted[i] = a;
    }
}

// Accepted candidates past the first `need` give their cell back; contested
// marks are cleared so the next batch starts from an empty contested map.
__global__ void finish_kernel(const uint64_t* __restrict__ cpos, int64_t T, const int32_t* __restrict__ accepted,
                              const int32_t* __restrict__ trank, const int32_t* __restrict__ cflag, int64_t need,
                              uint32_t* __restrict__ occ_bm, uint32_t* __restrict__ con_bm)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < T; i += (int64_t)gridDim.x * blockDim.x) {
        const bool give_back = accepted[i] && (int64_t)trank[i] >= need;
        const bool contested = cflag[i] != 0;
        if (!give_back && !contested) continue;
        const uint64_t p = cpos[i];
        const uint32_t bit = 1u << (p & 31);
        if (give_back) atomicAnd(&occ_bm[p >> 5], ~bit);
        if (contested) atomicAnd(&con_bm[p >> 5], ~bit);
    }
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

__device__ inline int32_t wave_incl(int32_t v)
{
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int32_t o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
}

__device__ inline int32_t wave_sum(int32_t v)
{
#pragma unroll
    for (int d = kWave / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
    return v;
}

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

template <bool DIRECT, bool WIDE>
__global__ void __launch_bounds__(kEmitThreads) emit_units_kernel(
    const uint32_t* __restrict__ occ_bm, const uint32_t* __restrict__ kept_bm, const uint32_t* __restrict__ old_bm,
    int64_t words, int64_t units, const int32_t* __restrict__ occ_cnt, const int32_t* __restrict__ old_cnt,
    const float* __restrict__ vold, int64_t nnz, int32_t K, int32_t* __restrict__ rows, int32_t* __restrict__ cols,
    float* __restrict__ vals)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t u = (int64_t)blockIdx.x * (kEmitThreads / kWave) + threadIdx.x / kWave;
    // the workgroup's four units share one prefix: all threads sum the counts
    // of the units before the workgroup, each wave then adds its neighbours'
    __shared__ int32_t red[2][kEmitThreads / kWave];
    const int64_t u0 = (int64_t)blockIdx.x * (kEmitThreads / kWave);
    int64_t run_o, run_d;
    if constexpr (DIRECT) {
        int32_t a = 0, b = 0;
        for (int64_t i = threadIdx.x; i < u0; i += kEmitThreads) {
            a += occ_cnt[i];
            b += old_cnt[i];
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
    if (u >= units) return;
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
        int64_t out = run_o + ia - a;
        const int64_t oldbase = run_d + ib - b;
        run_o += __shfl(ia, kWave - 1, kWave);
        run_d += __shfl(ib, kWave - 1, kWave);
        if (!om) continue;
        int64_t r, c;
        if constexpr (WIDE) {
            const uint64_t p0 = (uint64_t)w << 5;
            r = (int64_t)(p0 / (uint64_t)K);
            c = (int64_t)(p0 - (uint64_t)r * (uint64_t)K);
        } else {
            const uint32_t p0 = (uint32_t)w << 5;
            const uint32_t rr = p0 / (uint32_t)K;
            r = rr;
            c = (int64_t)(p0 - rr * (uint32_t)K);
        }
        int last = 0;
        uint32_t m = om;
        while (m && out < nnz) {
            const int bit = __ffs(m) - 1;
            m &= m - 1u;
            c += bit - last;
            last = bit;
            while (c >= K) {
                c -= K;
                ++r;
            }
            float v = 0.0f;
            if ((km >> bit) & 1u) v = vold[oldbase + __popc(dm & ((1u << bit) - 1u))];
            rows[out] = (int32_t)r;
            cols[out] = (int32_t)c;
            vals[out] = v;
            ++out;
        }
    }
}

struct PruneScratch {
    uint32_t* state;    // [16]
    int32_t* count;     // [4]
    uint32_t* hist;     // [256] selection histogram
    int32_t* tile_eq;   // [keep tiles] keys equal to T per tile (then their scan)
    float* vcopy;       // [nnz] the values before the rebuild
    uint32_t* kept_bm;  // [words]
    uint32_t* occ_bm;   // [words]
    uint32_t* old_bm;   // [words] cells of the entries before the drop
    uint32_t* con_bm;   // [words] contested cells of the current batch
    int32_t* occ_cnt;   // [units] occupied bits per emit unit (then their scan)
    int32_t* old_cnt;   // [units] old bits per emit unit
    uint64_t* cpos;     // [Tm]
    int32_t* acc;       // [Tm]
    int32_t* trank;     // [Tm]
    int32_t* cflag;     // [Tm] candidate names a contested cell
    unsigned long long* tab;   // [2^kHashBits]
    void* scan;         // scan scratch
    int64_t tmax, words, units, ktiles;
};

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
    const int64_t H = (int64_t)1 << kHashBits;
    int64_t sn = tm > units ? tm : units;
    if (ktiles > sn) sn = ktiles;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += al(bytes);
        return o;
    };
    size_t o_state = take(16 * 4), o_count = take(16), o_hist = take((size_t)256 * 4);
    size_t o_teq = take((size_t)ktiles * 4), o_vc = take((size_t)n * 4);
    size_t o_kbm = take((size_t)words * 4), o_obm = take((size_t)words * 4), o_dbm = take((size_t)words * 4);
    size_t o_cbm = take((size_t)words * 4);
    size_t o_oc = take((size_t)units * 4), o_dc = take((size_t)units * 4);
    size_t o_cpos = take((size_t)tm * 8), o_acc = take((size_t)tm * 4), o_trank = take((size_t)tm * 4);
    size_t o_cflag = take((size_t)tm * 4);
    size_t o_tab = take((size_t)H * 8);
    size_t o_scan = take(scan_scratch_bytes(sn));
    if (ps) {
        char* base = (char*)L->scratch;
        ps->state = (uint32_t*)(base + o_state);
        ps->count = (int32_t*)(base + o_count);
        ps->hist = (uint32_t*)(base + o_hist);
        ps->tile_eq = (int32_t*)(base + o_teq);
        ps->vcopy = (float*)(base + o_vc);
        ps->kept_bm = (uint32_t*)(base + o_kbm);
        ps->occ_bm = (uint32_t*)(base + o_obm);
        ps->old_bm = (uint32_t*)(base + o_dbm);
        ps->con_bm = (uint32_t*)(base + o_cbm);
        ps->occ_cnt = (int32_t*)(base + o_oc);
        ps->old_cnt = (int32_t*)(base + o_dc);
        ps->cpos = (uint64_t*)(base + o_cpos);
        ps->acc = (int32_t*)(base + o_acc);
        ps->trank = (int32_t*)(base + o_trank);
        ps->cflag = (int32_t*)(base + o_cflag);
        ps->tab = (unsigned long long*)(base + o_tab);
        ps->scan = base + o_scan;
        ps->tmax = tm;
        ps->words = words;
        ps->units = units;
        ps->ktiles = ktiles;
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

    // ---- drop: the n_drop-th smallest magnitude key T and its tie rank ----
    {
        const uint32_t init[3] = {0u, (uint32_t)(n_drop - 1), 0u};
        SNACK_HIP(hipMemcpyAsync(ps.state, init, sizeof init, hipMemcpyHostToDevice, s));
        int nblk = (int)grid_for(nnz);
        if (nblk > kSelBlocks) nblk = kSelBlocks;
        hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(kThreads), 0, s, ps.hist, (int64_t)256, 0u);
        for (int shift = 24; shift >= 0; shift -= 8) {
            hipLaunchKernelGGL(sel_hist_kernel, dim3(nblk), dim3(kThreads), 0, s, L->vals, nnz, ps.state, shift,
                               ps.hist);
            hipLaunchKernelGGL(sel_pick_kernel, dim3(1), dim3(256), 0, s, ps.hist, ps.state, shift);
        }
        SNACK_HIP(hipGetLastError());
        hipLaunchKernelGGL(eq_tiles_kernel, dim3((unsigned)ps.ktiles), dim3(kKeepThreads), 0, s, L->vals, nnz,
                           ps.state, ps.tile_eq);
        hipLaunchKernelGGL(zero4_kernel, dim3(grid_for(ps.words)), dim3(kThreads), 0, s, ps.kept_bm, ps.occ_bm,
                           ps.old_bm, ps.con_bm, ps.words);
        SNACK_HIP(hipGetLastError());
        if (ps.ktiles <= kKeepDirect) {
            hipLaunchKernelGGL(keep_tiles_kernel<true>, dim3((unsigned)ps.ktiles), dim3(kKeepThreads), 0, s, L->rows,
                               L->cols, L->vals, nnz, L->K, ps.state, ps.tile_eq, ps.vcopy, ps.kept_bm, ps.occ_bm,
                               ps.old_bm);
        } else {
            // a scan of zeros when every tie is dropped (the counts were not written then; they are not used)
            SNACK_CHECK(exclusive_scan_i32(ps.tile_eq, ps.tile_eq, ps.ktiles, nullptr, ps.scan, s));
            hipLaunchKernelGGL(keep_tiles_kernel<false>, dim3((unsigned)ps.ktiles), dim3(kKeepThreads), 0, s, L->rows,
                               L->cols, L->vals, nnz, L->K, ps.state, ps.tile_eq, ps.vcopy, ps.kept_bm, ps.occ_bm,
                               ps.old_bm);
        }
        SNACK_HIP(hipGetLastError());
    }

    // ---- grow: walk the candidate stream in batches ----
    int64_t need = n_drop;
    int64_t got = 0;
    uint64_t t0 = 0;
    int batches = 0;
    const int64_t H = (int64_t)1 << kHashBits;
    while (need > 0) {
        const double p_empty = (double)(N - (uint64_t)kept - (uint64_t)got) / (double)N;
        double want = (double)need / (p_empty > 1e-9 ? p_empty : 1e-9) * 1.03 + 4096.0;
        int64_t T = want > (double)ps.tmax ? ps.tmax : (int64_t)want;
        if (T < 1) T = 1;
        hipLaunchKernelGGL(gen_candidates_kernel, dim3(grid_for(T)), dim3(kThreads), 0, s, L->seed, L->epoch, t0, T, N,
                           ps.occ_bm, ps.cpos);
        hipLaunchKernelGGL(hash_clear_kernel, dim3(grid_for(H)), dim3(kThreads), 0, s, ps.tab, H);
        hipLaunchKernelGGL(claim_kernel, dim3(grid_for(T)), dim3(kThreads), 0, s, ps.cpos, T, N, ps.occ_bm, ps.con_bm);
        hipLaunchKernelGGL(contest_kernel, dim3(grid_for(T)), dim3(kThreads), 0, s, ps.cpos, T, N, ps.con_bm, ps.tab,
                           ps.cflag);
        hipLaunchKernelGGL(accept_kernel, dim3(grid_for(T)), dim3(kThreads), 0, s, ps.cpos, T, N, ps.cflag, ps.tab,
                           ps.acc);
        SNACK_HIP(hipGetLastError());
        SNACK_CHECK(exclusive_scan_i32(ps.acc, ps.trank, T, ps.count, ps.scan, s));
        hipLaunchKernelGGL(finish_kernel, dim3(grid_for(T)), dim3(kThreads), 0, s, ps.cpos, T, ps.acc, ps.trank,
                           ps.cflag, need, ps.occ_bm, ps.con_bm);
        SNACK_HIP(hipGetLastError());
        int32_t total = 0;
        SNACK_HIP(hipMemcpyAsync(&total, ps.count, 4, hipMemcpyDeviceToHost, s));
        SNACK_HIP(hipStreamSynchronize(s));
        const int64_t accepted = total < need ? total : need;
        got += accepted;
        need -= accepted;
        t0 += (uint64_t)T;
        if (++batches > 100000) return SNACK_ERR_UNSUPPORTED;
    }

    // ---- new canonical arrays: set bits of occ in ascending position ----
    {
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
            hipLaunchKernelGGL(kernel, dim3(grid), dim3(kEmitThreads), 0, s, ps.occ_bm, ps.kept_bm, ps.old_bm,
                               ps.words, nu, ps.occ_cnt, ps.old_cnt, ps.vcopy, nnz, L->K, L->rows, L->cols, L->vals);
        };
        if (direct) {
            if (wide) emit(emit_units_kernel<true, true>);
            else emit(emit_units_kernel<true, false>);
        } else {
            if (wide) emit(emit_units_kernel<false, true>);
            else emit(emit_units_kernel<false, false>);
        }
        SNACK_HIP(hipGetLastError());
    }
    SNACK_CHECK(canon_build_index(L, s));
    L->epoch += 1;
    return SNACK_OK;
}

}  // namespace snack
