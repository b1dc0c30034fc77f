// rows.hip -- row-local drop / regrow: every row keeps its number of entries.
// The "Padded-CSR" post (section 8.3) notes that SparseLab's SET and RigL keep
// each row's nnz fixed (only adaptive-density variants change it): the drop
// and the regrow both happen inside each row.  Row i with n_i entries drops
// d_i = floor(n_i * num / den) of them -- its smallest |v|, order key (IEEE
// bits of |v|, slot) -- and grows d_i cells of the same row that are empty
// after its drop, value +0.0:
//   random (SET)    candidate t of row i is the column high64(u_t * K), u_t the
//                   SplitMix64 output mix (Steele, Lea & Flood 2014) of
//                   s_i + (t + 1) * gamma, s_i = mix(seed ^ mix(epoch * 2^32 +
//                   i)); a candidate is accepted when its cell is neither kept
//                   nor accepted at a smaller t.  Candidates t < 64 K + 4096
//                   are tried; grows still missing after them take the
//                   smallest empty columns in order.
//   gradient (RigL) the d_i empty cells of largest |g|, g = sum_b dY[b, i]
//                   X[b, c] in fp32 with one fused multiply-add per batch row
//                   in batch order (a NaN counts as 0), ties by smaller column.
// These kernels write only the occupancy bitmaps of the global drop / regrow
// (`old`: cells before, `kept`: cells kept, `occ`: kept or grown) and the copy
// of the values; the canonical order and the column view are then rebuilt
// from them by the same code as there.
//
// drop (and random grow): one wavefront per row, the row's bitmap words in
//   LDS.  The d_i-th smallest magnitude is found by a radix select over the
//   row's entries (four digit passes, most significant first, histograms
//   added once per distinct digit of the wavefront), the ties at it are
//   dropped in slot order.  Random candidates are taken 64 at a time: while
//   the free ones cannot complete the row they are all claimed by atomic ORs
//   on the LDS words (a cell claimed twice counts once, whichever lane wins);
//   the chunk that can complete it ranks its first occurrences in t order.
//   Bitmap words lying wholly inside the row are stored; the words shared
//   with a neighbouring row (cleared beforehand) are combined with atomic ORs.
// gradient grow: one workgroup per 16 rows; every column's 16 scores are
//   fused multiply-add chains whose dY operands are uniform (scalar loads).
//   Four passes histogram the order key digit by digit per row among its
//   empty cells, a wavefront picks each row's digit from the top; a fifth
//   pass sets the cells above each row's threshold and ranks its ties in
//   column order.  The scores are recomputed in every pass: nothing of size
//   M*K is stored.
#include "internal.h"

namespace snack {
namespace {

constexpr uint64_t kRowGamma = 0x9E3779B97F4A7C15ull;

__device__ inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ inline uint32_t mag_key(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

__device__ inline uint32_t grad_key(float g) { return g != g ? 0u : (__float_as_uint(g) & 0x7FFFFFFFu); }

__device__ inline int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

__device__ inline uint64_t lanes_below() { return (1ull << lane_id()) - 1ull; }

// LDS written by some lanes of a wavefront is read by others afterwards
__device__ inline void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
}

__device__ inline uint32_t wave_incl_u32(uint32_t v)
{
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const uint32_t o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
}

// Adds one to h[dig] for every active lane: one LDS add per distinct digit of
// the wavefront (the loop runs the same number of times in every lane).
__device__ inline void hist_add(uint32_t* h, bool act, uint32_t dig)
{
    uint64_t m = __ballot(act);
    while (m) {
        const int l = __builtin_ctzll(m);
        const uint32_t dl = (uint32_t)__builtin_amdgcn_readlane((int)dig, l);
        const uint64_t same = __ballot(act && dig == dl);
        if (lane_id() == l) atomicAdd(&h[dl], (uint32_t)__popcll(same));
        if (dig == dl) act = false;
        m &= ~same;
    }
}

// The digit of a 256-bin histogram (bins counted from the smallest digit up
// when ASC, else from the largest down) that holds the rank-th key (1-based),
// and the rank within that digit.  Every lane returns the same pair.
template <bool ASC>
__device__ inline void pick_digit(const uint32_t* h, uint32_t rank, uint32_t& digit, uint32_t& rest,
                                  uint32_t* total = nullptr)
{
    const int lane = lane_id();
    uint32_t c[4], t[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        t[j] = ASC ? (uint32_t)(4 * lane + j) : (uint32_t)(255 - 4 * lane - j);
        c[j] = h[t[j]];
    }
    const uint32_t s = c[0] + c[1] + c[2] + c[3];
    const uint32_t inc = wave_incl_u32(s);
    const uint64_t hit = __ballot(inc >= rank);
    const int L = hit ? __builtin_ctzll(hit) : kWave - 1;
    uint32_t r = rank - (inc - s), d = t[3];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (r <= c[j]) {
            d = t[j];
            break;
        }
        r -= c[j];
    }
    digit = (uint32_t)__builtin_amdgcn_readlane((int)d, L);
    rest = (uint32_t)__builtin_amdgcn_readlane((int)r, L);
    if (total) *total = (uint32_t)__builtin_amdgcn_readlane((int)inc, kWave - 1);
}

struct RowArgs {
    const int32_t* row_ptr;
    const int32_t* cols;
    const float* vals;
    float* vcopy;
    uint32_t* old_bm;
    uint32_t* kept_bm;
    uint32_t* occ_bm;
    int32_t M, K;
    int64_t num, den;
    uint64_t seed, epoch;
    int32_t rw;   // LDS words of one row's bitmap
};

// The words that hold a row boundary (a row's first and last cell) may be
// shared by two rows: they are cleared here and combined by atomic ORs.
__global__ void row_edges_kernel(int32_t M, int32_t K, uint32_t* __restrict__ old_bm, uint32_t* __restrict__ kept_bm,
                                 uint32_t* __restrict__ occ_bm)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < M; i += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t a = ((uint64_t)i * (uint64_t)K) >> 5, b = (((uint64_t)i + 1) * (uint64_t)K - 1) >> 5;
        old_bm[a] = 0u;
        kept_bm[a] = 0u;
        occ_bm[a] = 0u;
        old_bm[b] = 0u;
        kept_bm[b] = 0u;
        occ_bm[b] = 0u;
    }
}

// store the row's words: those wholly inside the row directly, the others by OR
__device__ inline void put_row_words(uint32_t* __restrict__ bm, const uint32_t* w, uint64_t wa, int span,
                                     uint64_t first_cell, uint64_t end_cell)
{
    for (int q = lane_id(); q < span; q += kWave) {
        const uint64_t gw = wa + (uint64_t)q;
        const bool inside = gw * 32 >= first_cell && gw * 32 + 32 <= end_cell;
        const uint32_t v = w[q];
        if (inside) bm[gw] = v;
        else if (v) atomicOr(&bm[gw], v);
    }
}

template <bool SET>
__global__ void __launch_bounds__(256) row_drop_kernel(RowArgs a)
{
    extern __shared__ uint32_t lds[];
    const int waves = (int)(blockDim.x / kWave);
    const int wv = (int)(threadIdx.x / kWave);
    const int lane = lane_id();
    uint32_t* hist = lds + (size_t)wv * (256 + 2 * (size_t)a.rw);
    uint32_t* oldw = hist + 256;
    uint32_t* occw = oldw + a.rw;
    const uint64_t K = (uint64_t)a.K;
    for (int64_t i = (int64_t)blockIdx.x * waves + wv; i < a.M; i += (int64_t)gridDim.x * waves) {
        const int32_t p0 = a.row_ptr[i], p1 = a.row_ptr[i + 1];
        const int32_t n = p1 - p0;
        const int64_t d = (int64_t)n * a.num / a.den;
        const uint64_t first = (uint64_t)i * K, end = first + K;
        const uint64_t wa = first >> 5;
        const int span = (int)(((end - 1) >> 5) - wa) + 1;
        for (int q = lane; q < span; q += kWave) {
            oldw[q] = 0u;
            occw[q] = 0u;
        }
        wave_lds_sync();
        // ---- the drop threshold: T, and how many keys equal to T leave ----
        uint32_t T = 0u, ties = 0u;   // d == 0: nothing is below T = 0 and no tie leaves
        if (d == n && n > 0) {
            T = 0xFFFFFFFFu;          // every key is below
        } else if (d > 0) {
            uint32_t prefix = 0u, rank = (uint32_t)d;
#pragma unroll 1
            for (int pass = 0; pass < 4; ++pass) {
                const int shift = 24 - 8 * pass;
                for (int q = lane; q < 256; q += kWave) hist[q] = 0u;
                wave_lds_sync();
                for (int32_t b0 = p0; b0 < p1; b0 += kWave) {
                    const int32_t j = b0 + lane;
                    const bool in = j < p1;
                    const uint32_t m = in ? mag_key(a.vals[j]) : 0u;
                    const bool match = in && (pass == 0 || (m >> (shift + 8 < 32 ? shift + 8 : 31)) == prefix);
                    hist_add(hist, match, (m >> shift) & 0xFFu);
                }
                wave_lds_sync();
                uint32_t dig, rest;
                pick_digit<true>(hist, rank, dig, rest);
                prefix = (prefix << 8) | dig;
                rank = rest;
                wave_lds_sync();   // the histogram is read before the next pass clears it
            }
            T = prefix;
            ties = rank;
        }
        // ---- mark: old gets every entry, kept (in occw) the kept ones; copy the values ----
        uint32_t run = 0u;
        for (int32_t b0 = p0; b0 < p1; b0 += kWave) {
            const int32_t j = b0 + lane;
            const bool in = j < p1;
            const float v = in ? a.vals[j] : 0.0f;
            const int32_t c = in ? a.cols[j] : 0;
            const uint32_t m = mag_key(v);
            const bool tie = in && m == T;
            const uint64_t tm = __ballot(tie);
            const uint32_t tr = run + (uint32_t)__popcll(tm & lanes_below());
            run += (uint32_t)__popcll(tm);
            const bool drop = m < T || (tie && tr < ties);
            if (in) {
                a.vcopy[j] = v;
                const uint64_t lb = first + (uint64_t)c - (wa << 5);
                const uint32_t bit = 1u << (lb & 31);
                atomicOr(&oldw[lb >> 5], bit);
                if (!drop) atomicOr(&occw[lb >> 5], bit);
            }
        }
        wave_lds_sync();
        put_row_words(a.old_bm, oldw, wa, span, first, end);
        put_row_words(a.kept_bm, occw, wa, span, first, end);
        if constexpr (!SET) {
            put_row_words(a.occ_bm, occw, wa, span, first, end);
        } else {
            // ---- random grow inside the row ----
            int64_t need = d;
            const uint64_t s = mix64(a.seed ^ mix64((a.epoch << 32) + (uint64_t)i));
            const uint64_t tmax = 64ull * K + 4096ull;
            for (uint64_t t0 = 0; need > 0 && t0 < tmax; t0 += kWave) {
                const uint64_t t = t0 + (uint64_t)lane;
                const bool in = t < tmax;
                const uint64_t u = mix64(s + (t + 1ull) * kRowGamma);
                const uint32_t c = (uint32_t)__umul64hi(u, K);
                const uint64_t lb = first + c - (wa << 5);
                const uint32_t bit = 1u << (lb & 31);
                const bool fr = in && !(occw[lb >> 5] & bit);
                const uint64_t fm = __ballot(fr);
                if ((int64_t)__popcll(fm) < need) {
                    // the free candidates cannot complete the row: every distinct one is taken
                    bool took = false;
                    if (fr) took = !(atomicOr(&occw[lb >> 5], bit) & bit);
                    need -= (int64_t)__popcll(__ballot(took));
                } else {
                    // this chunk can complete the row: first occurrences in t order
                    bool firstocc = fr;
                    for (int q = 0; q < kWave - 1; ++q) {
                        if (!((fm >> q) & 1ull)) continue;
                        const uint32_t cq = (uint32_t)__builtin_amdgcn_readlane((int)c, q);
                        if (q < lane && cq == c) firstocc = false;
                    }
                    const uint64_t am = __ballot(firstocc);
                    const bool take = firstocc && (int64_t)__popcll(am & lanes_below()) < need;
                    if (take) atomicOr(&occw[lb >> 5], bit);
                    need -= (int64_t)__popcll(__ballot(take));
                }
                wave_lds_sync();
            }
            // the stream's bound reached: the smallest empty columns
            for (uint32_t c0 = 0; need > 0 && c0 < (uint32_t)K; c0 += kWave) {
                const uint32_t c = c0 + (uint32_t)lane;
                const bool in = c < (uint32_t)K;
                const uint64_t lb = first + (in ? c : 0u) - (wa << 5);
                const uint32_t bit = 1u << (lb & 31);
                const bool fr = in && !(occw[lb >> 5] & bit);
                const uint64_t fm = __ballot(fr);
                const bool take = fr && (int64_t)__popcll(fm & lanes_below()) < need;
                if (take) atomicOr(&occw[lb >> 5], bit);
                need -= (int64_t)__popcll(__ballot(take));
                wave_lds_sync();
            }
            put_row_words(a.occ_bm, occw, wa, span, first, end);
        }
        wave_lds_sync();   // the row's words are read before the next row clears them
    }
}

// ---- gradient grow --------------------------------------------------------
constexpr int kGR = 8;           // rows per workgroup
constexpr int kGThreadsR = 256;  // one column per thread and chunk
constexpr int kGWaves = kGThreadsR / kWave;
constexpr int kGB = 8;           // batch rows whose operands are loaded together

struct RowGradArgs {
    const float* X;
    const float* dY;
    int32_t B, M, K;
    const int32_t* row_ptr;
    int64_t num, den;
    const uint32_t* kept_bm;
    uint32_t* occ_bm;
};

// NB batch rows of the 16 score chains of a column: their X operands are
// loaded before any is used (the dY operands are uniform: scalar loads)
template <bool FULL, int NB>
__device__ inline void score_group(const RowGradArgs& a, int32_t r0, const float* __restrict__ xp, int32_t b,
                                   float (&acc)[kGR])
{
    const int32_t last = a.M - 1 - r0;
    float x[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) x[j] = xp[(int64_t)(b + j) * a.K];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const float* __restrict__ dy = a.dY + (int64_t)(b + j) * a.M + r0;
#pragma unroll
        for (int i = 0; i < kGR; ++i) acc[i] = fmaf(dy[FULL ? i : (i < last ? i : last)], x[j], acc[i]);
    }
}

// the 16 scores of column c: acc[i] = sum_b dY[b, r0 + i] X[b, c], one fused
// multiply-add per b in batch order (rows past M repeat the last row)
template <bool FULL>
__device__ inline void col_scores(const RowGradArgs& a, int32_t r0, int32_t c, float (&acc)[kGR])
{
#pragma unroll
    for (int i = 0; i < kGR; ++i) acc[i] = 0.0f;
    const float* __restrict__ xp = a.X + c;
    int32_t b = 0;
    for (; b + kGB <= a.B; b += kGB) score_group<FULL, kGB>(a, r0, xp, b, acc);
    if (a.B - b >= 4) {
        score_group<FULL, 4>(a, r0, xp, b, acc);
        b += 4;
    }
    if (a.B - b >= 2) {
        score_group<FULL, 2>(a, r0, xp, b, acc);
        b += 2;
    }
    if (a.B - b >= 1) score_group<FULL, 1>(a, r0, xp, b, acc);
}

__device__ inline bool kept_at(const uint32_t* __restrict__ bm, uint64_t p) { return (bm[p >> 5] >> (p & 31)) & 1u; }

// the words of the kept bitmap holding column c of the 16 rows (rows past M
// read row M - 1), and the bits taken out of them once they have arrived
template <bool FULL>
__device__ inline void kept_words(const uint32_t* __restrict__ bm, int32_t r0, int32_t M, uint64_t K, int32_t c,
                                  uint32_t (&w)[kGR])
{
#pragma unroll
    for (int i = 0; i < kGR; ++i) {
        const int32_t r = FULL ? r0 + i : (r0 + i < M ? r0 + i : M - 1);
        w[i] = bm[((uint64_t)r * K + (uint64_t)c) >> 5];
    }
}

template <bool FULL>
__device__ inline uint32_t kept_bits(const uint32_t (&w)[kGR], int32_t r0, int32_t M, uint64_t K, int32_t c)
{
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < kGR; ++i) {
        const int32_t r = FULL ? r0 + i : (r0 + i < M ? r0 + i : M - 1);
        const uint32_t bit = ((uint32_t)r * (uint32_t)K + (uint32_t)c) & 31u;   // low bits of the cell index
        m |= ((w[i] >> bit) & 1u) << i;
    }
    return m;
}

constexpr int kGS = 512;                  // sampled columns per row (at most)
constexpr uint32_t kOccupied = 0xFFFFFFFFu;  // sample entry of a cell that is not empty

struct RowGradLds {
    union {
        uint32_t hist[kGR][257];    // digit histograms of the passes
        uint32_t samp[kGR][kGS];    // keys of the sampled cells
    };
    uint32_t whist[kGWaves][256];   // one wavefront's histogram of the sample selection
    uint32_t need[kGR], pref[kGR], run[kGR], lo[kGR];
    uint32_t base[kGR], span[kGR];   // the key range a pass counts (emit: the lowest key set, and the shift)
    int32_t live[kGR];
    int32_t shift[kGR];   // the digits picked so far are key >> shift
    int32_t open[kGR];    // the row's threshold is not yet resolved
    int32_t first[kGR];   // the first digit is not yet picked
    int32_t d[kGR];
    int64_t e[kGR];       // empty cells of the row
    uint64_t ties[2][kGWaves][kGR];   // per chunk, wavefront and row: the lanes holding a cell at the threshold
};

// The rank-th largest (1-based) of the non-occupied keys in a row of the
// sample: a radix select by one wavefront.
__device__ inline uint32_t sample_select(const uint32_t* samp, int S, uint32_t rank, uint32_t* h)
{
    const int lane = lane_id();
    uint32_t prefix = 0u;
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int q = lane; q < 256; q += kWave) h[q] = 0u;
        wave_lds_sync();
        for (int j0 = 0; j0 < S; j0 += kWave) {
            const int j = j0 + lane;
            const uint32_t k = j < S ? samp[j] : kOccupied;
            const bool in = k != kOccupied && (pass == 0 || (k >> (shift + 8 < 32 ? shift + 8 : 31)) == prefix);
            hist_add(h, in, (k >> shift) & 0xFFu);
        }
        wave_lds_sync();
        uint32_t dig, rest;
        pick_digit<false>(h, rank, dig, rest);
        prefix = (prefix << 8) | dig;
        rank = rest;
        wave_lds_sync();
    }
    return prefix;
}

// The first digit pass over the row block: the top digit of every empty cell
// at or above the row's bound.  It meets cells of nearly every row in every
// chunk, so the kept words are loaded with the operands.  Without a bound
// (every cell counts) a wavefront's keys carry few distinct top digits: one
// add per digit; above a bound only a few lanes count: one add per lane.
template <bool FULL>
__device__ void sweep_first(const RowGradArgs& a, int32_t r0, RowGradLds& sh)
{
    const int tid = (int)threadIdx.x;
    const uint64_t K = (uint64_t)a.K;
    // the rows' parameters, uniform for the whole sweep (scalar registers)
    uint32_t live = 0u, bs[kGR];
#pragma unroll
    for (int i = 0; i < kGR; ++i) {
        bs[i] = (uint32_t)__builtin_amdgcn_readfirstlane((int)sh.base[i]);
        live |= (uint32_t)(__builtin_amdgcn_readfirstlane(sh.live[i]) != 0) << i;
    }
    for (int32_t c0 = 0; c0 < a.K; c0 += kGThreadsR) {
        const int32_t c = c0 + tid;
        const bool valid = c < a.K;
        const int32_t cc = valid ? c : 0;
        uint32_t kw[kGR];
        kept_words<FULL>(a.kept_bm, r0, a.M, K, cc, kw);
        float acc[kGR];
        col_scores<FULL>(a, r0, cc, acc);
        const uint32_t kept = kept_bits<FULL>(kw, r0, a.M, K, cc);
#pragma unroll
        for (int i = 0; i < kGR; ++i) {
            if (!((live >> i) & 1u)) continue;
            const uint32_t k = grad_key(acc[i]);
            const bool in = valid && k >= bs[i];
            if (!__ballot(in)) continue;
            const bool match = in && !((kept >> i) & 1u);
            if (bs[i] == 0u) hist_add(sh.hist[i], match, k >> 24);
            else if (match) atomicAdd(&sh.hist[i][k >> 24], 1u);
        }
    }
}

// A later digit pass: only the cells whose key has the row's prefix count.
// The second pass still meets a few cells of most rows in most chunks (the
// picked top digit spans two binades), so it loads the kept words with the
// operands; the later ones look a row's word up only when a lane has a cell.
template <bool FULL, bool UPFRONT>
__device__ void sweep_later(const RowGradArgs& a, int32_t r0, int shift, RowGradLds& sh)
{
    const int tid = (int)threadIdx.x;
    const uint64_t K = (uint64_t)a.K;
    uint32_t live = 0u, bs[kGR];
#pragma unroll
    for (int i = 0; i < kGR; ++i) {
        bs[i] = (uint32_t)__builtin_amdgcn_readfirstlane((int)sh.base[i]);
        live |= (uint32_t)(__builtin_amdgcn_readfirstlane(sh.live[i]) != 0) << i;
    }
    const uint32_t span = 1u << (shift + 8);
    for (int32_t c0 = 0; c0 < a.K; c0 += kGThreadsR) {
        const int32_t c = c0 + tid;
        const bool valid = c < a.K;
        const int32_t cc = valid ? c : 0;
        uint32_t kw[kGR];
        if (UPFRONT) kept_words<FULL>(a.kept_bm, r0, a.M, K, cc, kw);
        float acc[kGR];
        col_scores<FULL>(a, r0, cc, acc);
        const uint32_t kept = UPFRONT ? kept_bits<FULL>(kw, r0, a.M, K, cc) : 0u;
#pragma unroll
        for (int i = 0; i < kGR; ++i) {
            if (!((live >> i) & 1u)) continue;
            const uint32_t k = grad_key(acc[i]);
            const bool in = valid && k - bs[i] < span;
            if (!__ballot(in)) continue;
            if (in) {
                bool emp;
                if (UPFRONT) {
                    emp = !((kept >> i) & 1u);
                } else {
                    const uint64_t p = (uint64_t)(r0 + i) * K + (uint64_t)c;
                    emp = !kept_at(a.kept_bm, p);
                }
                if (emp) atomicAdd(&sh.hist[i][(k >> shift) & 0xFFu], 1u);
            }
        }
    }
}

// Per row: a sample of the row's columns gives a lower bound `lo` on its
// threshold (the sample key whose rank predicts about 4 d + 64 cells above
// it); the first digit pass counts only the cells at or above it, and a row
// whose bound was too high takes the first pass again without it.  After each
// digit pass the row's threshold is a prefix P of the key (key >> shift == P)
// and `need` cells with that prefix are still to be taken; when the prefix's
// whole bin is taken the row needs no further pass.  The emit pass sets the
// empty cells whose prefix is above P and the first `need` with prefix P in
// column order.  Every pass skips a row's chunk at once when no lane's key
// falls in the row's range.
template <bool FULL>
__device__ void row_grad_block(const RowGradArgs& a, int32_t r0, RowGradLds& sh)
{
    const int tid = (int)threadIdx.x, wv = tid / kWave, lane = lane_id();
    if (tid < kGR) {
        const int32_t r = r0 + tid;
        int64_t d = 0, n = 0;
        if (r < a.M) {
            n = a.row_ptr[r + 1] - a.row_ptr[r];
            d = n * a.num / a.den;
        }
        sh.d[tid] = (int32_t)d;
        sh.e[tid] = (int64_t)a.K - (n - d);
        sh.need[tid] = (uint32_t)d;
        sh.pref[tid] = 0u;
        sh.run[tid] = 0u;
        sh.lo[tid] = 0u;
        sh.shift[tid] = 31;
        sh.open[tid] = d > 0 ? 1 : 0;
        sh.first[tid] = d > 0 ? 1 : 0;
    }
    __syncthreads();
    int anyd = 0;
#pragma unroll
    for (int i = 0; i < kGR; ++i) anyd |= sh.d[i];
    if (!anyd) return;
    const uint64_t K = (uint64_t)a.K;

    // ---- the sample: columns j K / S, j < S ----
    const int S = a.K < kGS ? a.K : kGS;
    for (int j = tid; j < S; j += kGThreadsR) {
        const int32_t c = (int32_t)(((int64_t)j * a.K) / S);
        uint32_t kw[kGR];
        kept_words<FULL>(a.kept_bm, r0, a.M, K, c, kw);
        float acc[kGR];
        col_scores<FULL>(a, r0, c, acc);
        const uint32_t kept = kept_bits<FULL>(kw, r0, a.M, K, c);
#pragma unroll
        for (int i = 0; i < kGR; ++i) sh.samp[i][j] = ((kept >> i) & 1u) ? kOccupied : grad_key(acc[i]);
    }
    __syncthreads();
    for (int i = wv; i < kGR; i += kGWaves) {
        if (sh.d[i] <= 0) continue;
        uint32_t se = 0u;
        for (int j = lane; j < S; j += kWave) se += sh.samp[i][j] != kOccupied ? 1u : 0u;
        se = wave_incl_u32(se);
        se = (uint32_t)__builtin_amdgcn_readlane((int)se, kWave - 1);
        const int64_t want = 4 * (int64_t)sh.d[i] + 64;
        const int64_t r = (want * (int64_t)se + sh.e[i] - 1) / sh.e[i];
        uint32_t lo = 0u;
        if (r < (int64_t)se) lo = sample_select(sh.samp[i], S, (uint32_t)r, sh.whist[wv]);
        if (lane == 0) sh.lo[i] = lo;
    }
    __syncthreads();

    // ---- digit passes, most significant first (the first one at most twice) ----
#pragma unroll 1
    for (int pass = 0, round = 0; pass < 4;) {
        const int shift = 24 - 8 * pass;
        if (tid < kGR) {
            const int i = tid;
            sh.live[i] = sh.open[i] != 0 && (pass > 0 || sh.first[i] != 0);
            if (pass == 0) {
                sh.base[i] = sh.lo[i];
                sh.span[i] = 0x80000000u - sh.lo[i];
            } else {
                sh.base[i] = sh.pref[i] << (shift + 8);
                sh.span[i] = 1u << (shift + 8);
            }
        }
        __syncthreads();
        int any = 0;
#pragma unroll
        for (int i = 0; i < kGR; ++i) any |= sh.live[i];
        if (!any) {
            if (pass == 0) {   // no row (left) for the first pass
                pass = 1;
                round = 1;
                continue;
            }
            break;             // every row is resolved
        }
        for (int q = tid; q < kGR * 257; q += kGThreadsR) (&sh.hist[0][0])[q] = 0u;
        __syncthreads();
        if (pass == 0) sweep_first<FULL>(a, r0, sh);
        else if (pass == 1) sweep_later<FULL, true>(a, r0, shift, sh);
        else sweep_later<FULL, false>(a, r0, shift, sh);
        __syncthreads();
        for (int i = wv; i < kGR; i += kGWaves) {
            if (!sh.live[i]) continue;
            uint32_t dig, rest, total;
            pick_digit<false>(sh.hist[i], sh.need[i], dig, rest, &total);
            if (lane == 0) {
                if (total < sh.need[i]) {
                    sh.lo[i] = 0u;   // the bound was too high: the first pass again, over every cell
                } else {
                    sh.pref[i] = (sh.pref[i] << 8) | dig;
                    sh.need[i] = rest;
                    sh.shift[i] = shift;
                    sh.first[i] = 0;
                    // the whole bin is taken: done, unless cells below the bound share it
                    const bool whole = rest == sh.hist[i][dig] && (pass > 0 || sh.lo[i] == 0u ||
                                                                   (sh.lo[i] >> 24) < dig);
                    if (whole || pass == 3) sh.open[i] = 0;
                }
            }
        }
        __syncthreads();
        if (pass == 0 && round == 0) {
            round = 1;   // rows whose bound was too high take the first pass once more
        } else {
            ++pass;
        }
    }
    // ---- set the cells above each row's threshold and the first `need` at it ----
    if (tid < kGR) {
        sh.base[tid] = sh.pref[tid] << sh.shift[tid];
        sh.live[tid] = sh.d[tid] > 0;
    }
    __syncthreads();
    int par = 0;
    for (int32_t c0 = 0; c0 < a.K; c0 += kGThreadsR, par ^= 1) {
        const int32_t c = c0 + tid;
        const bool valid = c < a.K;
        const int32_t cc = valid ? c : 0;
        float acc[kGR];
        col_scores<FULL>(a, r0, cc, acc);
#pragma unroll
        for (int i = 0; i < kGR; ++i) {
            if (!sh.live[i]) continue;
            const uint32_t k = grad_key(acc[i]);
            bool in = valid && k >= sh.base[i];
            uint64_t tm = 0ull;
            if (__ballot(in)) {
                const uint64_t p = (uint64_t)(r0 + i) * K + (uint64_t)c;
                in = in && !kept_at(a.kept_bm, p);
                const uint32_t kp = k >> sh.shift[i];
                const uint32_t P = sh.pref[i];
                if (in && kp > P) atomicOr(&a.occ_bm[p >> 5], 1u << (p & 31));
                tm = __ballot(in && kp == P);
            }
            if (lane == 0) sh.ties[par][wv][i] = tm;
        }
        __syncthreads();
        // the cells at the threshold: their rank in column order decides
#pragma unroll 1
        for (int i = 0; i < kGR; ++i) {
            if (!sh.live[i]) continue;
            const uint64_t tm = sh.ties[par][wv][i];
            if (!tm) continue;
            uint32_t rank = sh.run[i];
            for (int w = 0; w < wv; ++w) rank += (uint32_t)__popcll(sh.ties[par][w][i]);
            rank += (uint32_t)__popcll(tm & lanes_below());
            if (((tm >> lane) & 1ull) && rank < sh.need[i]) {
                const uint64_t p = (uint64_t)(r0 + i) * K + (uint64_t)c;
                atomicOr(&a.occ_bm[p >> 5], 1u << (p & 31));
            }
        }
        __syncthreads();
        if (tid < kGR && sh.live[tid]) {
            uint32_t add = 0u;
            for (int w = 0; w < kGWaves; ++w) add += (uint32_t)__popcll(sh.ties[par][w][tid]);
            sh.run[tid] += add;
        }
    }
}

__global__ void __launch_bounds__(kGThreadsR)
row_grad_kernel(const float* __restrict__ X, const float* __restrict__ dY, const int32_t* __restrict__ row_ptr,
                const uint32_t* __restrict__ kept_bm, uint32_t* __restrict__ occ_bm, int32_t B, int32_t M, int32_t K,
                int64_t num, int64_t den)
{
    __shared__ RowGradLds sh;
    RowGradArgs a;
    a.X = X;
    a.dY = dY;
    a.row_ptr = row_ptr;
    a.kept_bm = kept_bm;
    a.occ_bm = occ_bm;
    a.B = B;
    a.M = M;
    a.K = K;
    a.num = num;
    a.den = den;
    const int32_t r0 = (int32_t)blockIdx.x * kGR;
    if (r0 + kGR <= a.M) row_grad_block<true>(a, r0, sh);
    else row_grad_block<false>(a, r0, sh);
}

int row_words(int32_t K) { return (int)(((int64_t)K + 31) / 32 + 1); }

}  // namespace

int64_t rows_lds_per_wave(int32_t K) { return (int64_t)(256 + 2 * (int64_t)row_words(K)) * 4; }

snack_status rows_drop_grow(const RowDst& r, int lds_limit, hipStream_t s)
{
    if (r.M <= 0 || r.K <= 0) return SNACK_OK;
    const int64_t per = rows_lds_per_wave(r.K);
    int waves = 4;
    while (waves > 1 && per * waves > 65536) waves >>= 1;
    if (per * waves > lds_limit) return SNACK_ERR_UNSUPPORTED;
    RowArgs a;
    a.row_ptr = r.row_ptr;
    a.cols = r.cols;
    a.vals = r.vals;
    a.vcopy = r.vcopy;
    a.old_bm = r.old_bm;
    a.kept_bm = r.kept_bm;
    a.occ_bm = r.occ_bm;
    a.M = r.M;
    a.K = r.K;
    a.num = r.num;
    a.den = r.den;
    a.seed = r.seed;
    a.epoch = r.epoch;
    a.rw = row_words(r.K);
    {
        int64_t g = ((int64_t)r.M + 255) / 256;
        if (g > 4096) g = 4096;
        hipLaunchKernelGGL(row_edges_kernel, dim3((unsigned)g), dim3(256), 0, s, r.M, r.K, r.old_bm, r.kept_bm,
                           r.occ_bm);
    }
    {
        int64_t g = ((int64_t)r.M + waves - 1) / waves;
        if (g > (1 << 20)) g = 1 << 20;
        const size_t lds = (size_t)(per * waves);
        if (r.gradient)
            hipLaunchKernelGGL(row_drop_kernel<false>, dim3((unsigned)g), dim3(waves * kWave), lds, s, a);
        else
            hipLaunchKernelGGL(row_drop_kernel<true>, dim3((unsigned)g), dim3(waves * kWave), lds, s, a);
    }
    SNACK_HIP(hipGetLastError());
    if (r.gradient) {
        RowGradArgs g;
        g.X = r.X;
        g.dY = r.dY;
        g.B = r.B;
        g.M = r.M;
        g.K = r.K;
        g.row_ptr = r.row_ptr;
        g.num = r.num;
        g.den = r.den;
        g.kept_bm = r.kept_bm;
        g.occ_bm = r.occ_bm;
        const int64_t blocks = ((int64_t)r.M + kGR - 1) / kGR;
        hipLaunchKernelGGL(row_grad_kernel, dim3((unsigned)blocks), dim3(kGThreadsR), 0, s, g.X, g.dY, g.row_ptr,
                           g.kept_bm, g.occ_bm, g.B, g.M, g.K, g.num, g.den);
        SNACK_HIP(hipGetLastError());
    }
    return SNACK_OK;
}

}  // namespace snack
