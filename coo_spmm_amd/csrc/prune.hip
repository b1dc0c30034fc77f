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
// state: [0] prefix, [1] rank still to find among keys matching the prefix.
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
    }
}

__global__ void eq_flags_kernel(const float* __restrict__ vals, int64_t n, const uint32_t* __restrict__ state,
                                int32_t* __restrict__ eq)
{
    const uint32_t T = state[0];
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += (int64_t)gridDim.x * blockDim.x)
        eq[k] = mag_bits(vals[k]) == T ? 1 : 0;
}

// keep[k] = 0 for the dropped entries: key < T, or key == T among the first (rank+1) ties in slot order
__global__ void keep_flags_kernel(const float* __restrict__ vals, int64_t n, const uint32_t* __restrict__ state,
                                  const int32_t* __restrict__ eqrank, int32_t* __restrict__ keep)
{
    const uint32_t T = state[0];
    const uint32_t ties = state[1] + 1;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t key = mag_bits(vals[k]);
        const bool drop = key < T || (key == T && (uint32_t)eqrank[k] < ties);
        keep[k] = drop ? 0 : 1;
    }
}

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

__device__ inline uint64_t cell_of(const int32_t* __restrict__ rows, const int32_t* __restrict__ cols, int64_t k,
                                   int32_t K)
{
    return (uint64_t)rows[k] * (uint64_t)K + (uint64_t)cols[k];
}

// Kept values in canonical order, and the kept bitmap word by word: the first
// entry of each 32-cell word assembles the word from the entries that follow
// it (positions ascend, so they are adjacent), hence no atomics.  Both bitmaps
// start as the kept cells.  Bitmaps must be zero beforehand.
__global__ void kept_bits_kernel(const int32_t* __restrict__ rows, const int32_t* __restrict__ cols,
                                 const float* __restrict__ vals, int64_t n, int32_t K,
                                 const int32_t* __restrict__ keep, const int32_t* __restrict__ kidx,
                                 float* __restrict__ kval, uint32_t* __restrict__ kept_bm,
                                 uint32_t* __restrict__ occ_bm)
{
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += (int64_t)gridDim.x * blockDim.x) {
        if (keep[k]) kval[kidx[k]] = vals[k];
        const uint64_t p = cell_of(rows, cols, k, K);
        const uint64_t w = p >> 5;
        if (k > 0 && (cell_of(rows, cols, k - 1, K) >> 5) == w) continue;
        uint32_t m = 0;
        for (int64_t j = k; j < n; ++j) {
            const uint64_t q = j == k ? p : cell_of(rows, cols, j, K);
            if ((q >> 5) != w) break;
            if (keep[j]) m |= 1u << (q & 31);
        }
        if (m) {
            kept_bm[w] = m;
            occ_bm[w] = m;
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
// Tiles of 4096 bitmap words (256 threads x 16 consecutive words).  Kernel 1
// counts each tile's occupied and kept bits; kernel 2 gives every thread its
// first output slot and kept rank (the tile's prefix -- summed from the tile
// counts before it when there are few tiles, else read from their scans --
// plus a block scan of the thread counts) and emits its cells in order.
constexpr int kEmitThreads = 256;
constexpr int kEmitWords = 16;
constexpr int64_t kEmitTile = (int64_t)kEmitThreads * kEmitWords;
constexpr int64_t kEmitDirect = 4096;

__device__ inline void block_exclusive2(int32_t& a, int32_t& b, int32_t* smem /*[2 * waves]*/, int32_t& ta,
                                        int32_t& tb)
{
    constexpr int W = kEmitThreads / kWave;
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    int32_t ia = a, ib = b;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int32_t oa = __shfl_up(ia, d, kWave), ob = __shfl_up(ib, d, kWave);
        if (lane >= d) {
            ia += oa;
            ib += ob;
        }
    }
    if (lane == kWave - 1) {
        smem[w] = ia;
        smem[W + w] = ib;
    }
    __syncthreads();
    int32_t ba = 0, bb = 0;
    ta = 0;
    tb = 0;
#pragma unroll
    for (int i = 0; i < W; ++i) {
        const int32_t xa = smem[i], xb = smem[W + i];
        if (i < w) {
            ba += xa;
            bb += xb;
        }
        ta += xa;
        tb += xb;
    }
    __syncthreads();
    a = ba + ia - a;
    b = bb + ib - b;
}

__device__ inline void load_words(const uint32_t* __restrict__ bm, int64_t w0, int64_t words,
                                  uint32_t (&x)[kEmitWords])
{
#pragma unroll
    for (int q = 0; q < kEmitWords / 4; ++q) {
        const int64_t w = w0 + 4 * q;
        if (w + 3 < words) {
            const uint4 v = *reinterpret_cast<const uint4*>(bm + w);
            x[4 * q] = v.x;
            x[4 * q + 1] = v.y;
            x[4 * q + 2] = v.z;
            x[4 * q + 3] = v.w;
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) x[4 * q + t] = w + t < words ? bm[w + t] : 0u;
        }
    }
}

__global__ void __launch_bounds__(kEmitThreads) bm_tile_counts_kernel(const uint32_t* __restrict__ occ_bm,
                                                                      const uint32_t* __restrict__ kept_bm,
                                                                      int64_t words, int32_t* __restrict__ occ_sum,
                                                                      int32_t* __restrict__ kept_sum)
{
    __shared__ int32_t smem[2 * (kEmitThreads / kWave)];
    const int64_t w0 = (int64_t)blockIdx.x * kEmitTile + (int64_t)threadIdx.x * kEmitWords;
    uint32_t o[kEmitWords], k[kEmitWords];
    load_words(occ_bm, w0, words, o);
    load_words(kept_bm, w0, words, k);
    int32_t a = 0, b = 0;
#pragma unroll
    for (int j = 0; j < kEmitWords; ++j) {
        a += __popc(o[j]);
        b += __popc(k[j]);
    }
    int32_t ta, tb;
    block_exclusive2(a, b, smem, ta, tb);
    if (threadIdx.x == 0) {
        occ_sum[blockIdx.x] = ta;
        kept_sum[blockIdx.x] = tb;
    }
}

template <bool DIRECT>
__global__ void __launch_bounds__(kEmitThreads) emit_tiles_kernel(
    const uint32_t* __restrict__ occ_bm, const uint32_t* __restrict__ kept_bm, int64_t words,
    const int32_t* __restrict__ occ_sum, const int32_t* __restrict__ kept_sum, const float* __restrict__ kval,
    int64_t nnz, int64_t nkept, int32_t K, int32_t* __restrict__ rows, int32_t* __restrict__ cols,
    float* __restrict__ vals)
{
    __shared__ int32_t smem[2 * (kEmitThreads / kWave)];
    const int64_t tile = blockIdx.x;
    int32_t po, pk;
    if constexpr (DIRECT) {
        int32_t a = 0, b = 0;
        for (int64_t i = threadIdx.x; i < tile; i += kEmitThreads) {
            a += occ_sum[i];
            b += kept_sum[i];
        }
        block_exclusive2(a, b, smem, po, pk);
    } else {
        po = occ_sum[tile];
        pk = kept_sum[tile];
    }
    // the tile's words in kEmitWords sweeps of one word per thread: neighbouring
    // threads write neighbouring entries; the block scan gives each its slot
    int64_t run_o = po, run_k = pk;
    for (int it = 0; it < kEmitWords; ++it) {
        const int64_t w = tile * kEmitTile + (int64_t)it * kEmitThreads + threadIdx.x;
        const uint32_t om = w < words ? occ_bm[w] : 0u;
        const uint32_t km = w < words ? kept_bm[w] : 0u;
        int32_t a = __popc(om), b = __popc(km);
        int32_t ta, tb;
        block_exclusive2(a, b, smem, ta, tb);
        int64_t out = run_o + a;
        int64_t ki = run_k + b;
        run_o += ta;
        run_k += tb;
        if (!om) continue;
        const uint64_t p0 = (uint64_t)w << 5;
        int64_t r = (int64_t)(p0 / (uint64_t)K);
        int64_t c = (int64_t)(p0 - (uint64_t)r * (uint64_t)K);
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
            rows[out] = (int32_t)r;
            cols[out] = (int32_t)c;
            vals[out] = ((km >> bit) & 1u) && ki < nkept ? kval[ki++] : 0.0f;
            ++out;
        }
    }
}

struct PruneScratch {
    uint32_t* state;    // [16]
    int32_t* count;     // [4]
    uint32_t* selmat;   // [256] selection histogram
    int32_t* a;         // [nnz] flags / eq
    int32_t* b;         // [nnz] scan result
    int32_t* keep;      // [nnz]
    float* kval;        // [nnz]
    uint32_t* kept_bm;  // [words]
    uint32_t* occ_bm;   // [words]
    uint32_t* con_bm;   // [words] contested cells of the current batch
    int32_t* cflag;     // [Tm] candidate names a contested cell
    int32_t* occ_cnt;   // [tiles] occupied bits per emit tile (then their scan)
    int32_t* kept_cnt;  // [tiles] kept bits per emit tile
    uint64_t* cpos;     // [Tm]
    int32_t* acc;       // [Tm]
    int32_t* trank;     // [Tm]
    unsigned long long* tab;   // [2^kHashBits]
    void* scan;         // scan scratch
    int64_t tmax, words, groups;
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
    const int64_t groups = (words + kEmitTile - 1) / kEmitTile;
    const int64_t tm = batch_cap(L);
    const int64_t H = (int64_t)1 << kHashBits;
    int64_t sn = tm > n ? tm : n;
    if (groups > sn) sn = groups;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += al(bytes);
        return o;
    };
    size_t o_state = take(16 * 4), o_count = take(16), o_sel = take((size_t)256 * 4);
    size_t o_a = take((size_t)n * 4), o_b = take((size_t)n * 4), o_keep = take((size_t)n * 4);
    size_t o_kval = take((size_t)n * 4);
    size_t o_kbm = take((size_t)words * 4), o_obm = take((size_t)words * 4), o_cbm = take((size_t)words * 4);
    size_t o_oc = take((size_t)groups * 4), o_kc = take((size_t)groups * 4);
    size_t o_cpos = take((size_t)tm * 8), o_acc = take((size_t)tm * 4), o_trank = take((size_t)tm * 4);
    size_t o_cflag = take((size_t)tm * 4);
    size_t o_tab = take((size_t)H * 8);
    size_t o_scan = take(scan_scratch_bytes(sn));
    if (ps) {
        char* base = (char*)L->scratch;
        ps->state = (uint32_t*)(base + o_state);
        ps->count = (int32_t*)(base + o_count);
        ps->selmat = (uint32_t*)(base + o_sel);
        ps->a = (int32_t*)(base + o_a);
        ps->b = (int32_t*)(base + o_b);
        ps->keep = (int32_t*)(base + o_keep);
        ps->kval = (float*)(base + o_kval);
        ps->kept_bm = (uint32_t*)(base + o_kbm);
        ps->occ_bm = (uint32_t*)(base + o_obm);
        ps->con_bm = (uint32_t*)(base + o_cbm);
        ps->cflag = (int32_t*)(base + o_cflag);
        ps->occ_cnt = (int32_t*)(base + o_oc);
        ps->kept_cnt = (int32_t*)(base + o_kc);
        ps->cpos = (uint64_t*)(base + o_cpos);
        ps->acc = (int32_t*)(base + o_acc);
        ps->trank = (int32_t*)(base + o_trank);
        ps->tab = (unsigned long long*)(base + o_tab);
        ps->scan = base + o_scan;
        ps->tmax = tm;
        ps->words = words;
        ps->groups = groups;
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
        uint32_t init[2] = {0u, (uint32_t)(n_drop - 1)};
        SNACK_HIP(hipMemcpyAsync(ps.state, init, sizeof init, hipMemcpyHostToDevice, s));
        int nblk = (int)grid_for(nnz);
        if (nblk > kSelBlocks) nblk = kSelBlocks;
        hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(kThreads), 0, s, ps.selmat, (int64_t)256, 0u);
        for (int shift = 24; shift >= 0; shift -= 8) {
            hipLaunchKernelGGL(sel_hist_kernel, dim3(nblk), dim3(kThreads), 0, s, L->vals, nnz, ps.state, shift,
                               ps.selmat);
            hipLaunchKernelGGL(sel_pick_kernel, dim3(1), dim3(256), 0, s, ps.selmat, ps.state, shift);
        }
        SNACK_HIP(hipGetLastError());
        hipLaunchKernelGGL(eq_flags_kernel, dim3(grid_for(nnz)), dim3(kThreads), 0, s, L->vals, nnz, ps.state, ps.a);
        SNACK_CHECK(exclusive_scan_i32(ps.a, ps.b, nnz, nullptr, ps.scan, s));
        hipLaunchKernelGGL(keep_flags_kernel, dim3(grid_for(nnz)), dim3(kThreads), 0, s, L->vals, nnz, ps.state, ps.b,
                           ps.keep);
        SNACK_CHECK(exclusive_scan_i32(ps.keep, ps.b, nnz, nullptr, ps.scan, s));
        hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(ps.words)), dim3(kThreads), 0, s, ps.kept_bm, ps.words, 0u);
        hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(ps.words)), dim3(kThreads), 0, s, ps.occ_bm, ps.words, 0u);
        hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(ps.words)), dim3(kThreads), 0, s, ps.con_bm, ps.words, 0u);
        hipLaunchKernelGGL(kept_bits_kernel, dim3(grid_for(nnz)), dim3(kThreads), 0, s, L->rows, L->cols, L->vals,
                           nnz, L->K, ps.keep, ps.b, ps.kval, ps.kept_bm, ps.occ_bm);
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
        const int64_t nt = ps.groups;
        hipLaunchKernelGGL(bm_tile_counts_kernel, dim3((unsigned)nt), dim3(kEmitThreads), 0, s, ps.occ_bm, ps.kept_bm,
                           ps.words, ps.occ_cnt, ps.kept_cnt);
        SNACK_HIP(hipGetLastError());
        if (nt <= kEmitDirect) {
            hipLaunchKernelGGL(emit_tiles_kernel<true>, dim3((unsigned)nt), dim3(kEmitThreads), 0, s, ps.occ_bm,
                               ps.kept_bm, ps.words, ps.occ_cnt, ps.kept_cnt, ps.kval, nnz, kept, L->K, L->rows,
                               L->cols, L->vals);
        } else {
            SNACK_CHECK(exclusive_scan_i32(ps.occ_cnt, ps.occ_cnt, nt, nullptr, ps.scan, s));
            SNACK_CHECK(exclusive_scan_i32(ps.kept_cnt, ps.kept_cnt, nt, nullptr, ps.scan, s));
            hipLaunchKernelGGL(emit_tiles_kernel<false>, dim3((unsigned)nt), dim3(kEmitThreads), 0, s, ps.occ_bm,
                               ps.kept_bm, ps.words, ps.occ_cnt, ps.kept_cnt, ps.kval, nnz, kept, L->K, L->rows,
                               L->cols, L->vals);
        }
        SNACK_HIP(hipGetLastError());
    }
    SNACK_CHECK(canon_build_index(L, s));
    L->epoch += 1;
    return SNACK_OK;
}

}  // namespace snack
