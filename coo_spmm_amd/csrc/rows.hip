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
__device__ inline void pick_digit(const uint32_t* h, uint32_t rank, uint32_t& digit, uint32_t& rest)
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
constexpr int kGR = 16;          // rows per workgroup
constexpr int kGThreadsR = 256;  // one column per thread and chunk
constexpr int kGWaves = kGThreadsR / kWave;

struct RowGradArgs {
    const float* X;
    const float* dY;
    int32_t B, M, K;
    const int32_t* row_ptr;
    int64_t num, den;
    const uint32_t* kept_bm;
    uint32_t* occ_bm;
};

// the 16 scores of column c: acc[i] = sum_b dY[b, r0 + i] X[b, c], one fused
// multiply-add per b in batch order (rows past M repeat the last row)
template <bool FULL>
__device__ inline void col_scores(const RowGradArgs& a, int32_t r0, int32_t c, float (&acc)[kGR])
{
#pragma unroll
    for (int i = 0; i < kGR; ++i) acc[i] = 0.0f;
    const float* __restrict__ xp = a.X + c;
    const int32_t last = a.M - 1 - r0;
#pragma unroll 4
    for (int32_t b = 0; b < a.B; ++b) {
        const float x = xp[(int64_t)b * a.K];
        const float* __restrict__ dy = a.dY + (int64_t)b * a.M + r0;
#pragma unroll
        for (int i = 0; i < kGR; ++i) acc[i] = fmaf(dy[FULL ? i : (i < last ? i : last)], x, acc[i]);
    }
}

__device__ inline bool kept_at(const uint32_t* __restrict__ bm, uint64_t p) { return (bm[p >> 5] >> (p & 31)) & 1u; }

struct RowGradLds {
    uint32_t hist[kGR][257];
    uint32_t need[kGR], pref[kGR], run[kGR];
    int32_t d[kGR];
    uint32_t cnt[2][kGWaves][kGR];
};

template <bool FULL>
__device__ void row_grad_block(const RowGradArgs& a, int32_t r0, RowGradLds& sh)
{
    auto& hist = sh.hist;
    auto& s_need = sh.need;
    auto& s_pref = sh.pref;
    auto& s_run = sh.run;
    auto& s_d = sh.d;
    auto& s_cnt = sh.cnt;
    const int tid = (int)threadIdx.x, wv = tid / kWave, lane = lane_id();
    if (tid < kGR) {
        const int32_t r = r0 + tid;
        int64_t d = 0;
        if (r < a.M) d = (int64_t)(a.row_ptr[r + 1] - a.row_ptr[r]) * a.num / a.den;
        s_d[tid] = (int32_t)d;
        s_need[tid] = (uint32_t)d;
        s_pref[tid] = 0u;
        s_run[tid] = 0u;
    }
    __syncthreads();
    int any = 0;
#pragma unroll
    for (int i = 0; i < kGR; ++i) any |= s_d[i];
    if (!any) return;
    const uint64_t K = (uint64_t)a.K;
    // ---- four digit passes ----
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int q = tid; q < kGR * 257; q += kGThreadsR) (&hist[0][0])[q] = 0u;
        uint32_t pref[kGR];
        bool live[kGR];
#pragma unroll
        for (int i = 0; i < kGR; ++i) {
            pref[i] = s_pref[i];
            live[i] = s_d[i] > 0;
        }
        __syncthreads();
        for (int32_t c0 = 0; c0 < a.K; c0 += kGThreadsR) {
            const int32_t c = c0 + tid;
            const bool valid = c < a.K;
            float acc[kGR];
            col_scores<FULL>(a, r0, valid ? c : 0, acc);
#pragma unroll
            for (int i = 0; i < kGR; ++i) {
                if (!live[i]) continue;
                const uint32_t k = grad_key(acc[i]);
                const bool empty = valid && !kept_at(a.kept_bm, (uint64_t)(r0 + i) * K + (uint64_t)c);
                const bool match = empty && (pass == 0 || (k >> (shift + 8 < 32 ? shift + 8 : 31)) == pref[i]);
                hist_add(hist[i], match, (k >> shift) & 0xFFu);
            }
        }
        __syncthreads();
        for (int i = wv; i < kGR; i += kGWaves) {
            if (s_d[i] <= 0) continue;
            uint32_t dig, rest;
            pick_digit<false>(hist[i], s_need[i], dig, rest);
            if (lane == 0) {
                s_pref[i] = (s_pref[i] << 8) | dig;
                s_need[i] = rest;
            }
        }
        __syncthreads();
    }
    // ---- set the cells above each row's threshold and the first ties at it ----
    uint32_t T[kGR], take[kGR];
    bool live[kGR];
#pragma unroll
    for (int i = 0; i < kGR; ++i) {
        T[i] = s_pref[i];
        take[i] = s_need[i];
        live[i] = s_d[i] > 0;
    }
    int par = 0;
    for (int32_t c0 = 0; c0 < a.K; c0 += kGThreadsR, par ^= 1) {
        const int32_t c = c0 + tid;
        const bool valid = c < a.K;
        float acc[kGR];
        col_scores<FULL>(a, r0, valid ? c : 0, acc);
        uint64_t tm[kGR];
#pragma unroll
        for (int i = 0; i < kGR; ++i) {
            tm[i] = 0ull;
            if (!live[i]) continue;
            const uint32_t k = grad_key(acc[i]);
            const uint64_t p = (uint64_t)(r0 + i) * K + (uint64_t)c;
            const bool empty = valid && !kept_at(a.kept_bm, p);
            if (empty && k > T[i]) atomicOr(&a.occ_bm[p >> 5], 1u << (p & 31));
            tm[i] = __ballot(empty && k == T[i]);
            if (lane == 0) s_cnt[par][wv][i] = (uint32_t)__popcll(tm[i]);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kGR; ++i) {
            if (!tm[i]) continue;
            uint32_t rank = s_run[i];
            for (int w = 0; w < wv; ++w) rank += s_cnt[par][w][i];
            rank += (uint32_t)__popcll(tm[i] & lanes_below());
            if (((tm[i] >> lane) & 1ull) && rank < take[i]) {
                const uint64_t p = (uint64_t)(r0 + i) * K + (uint64_t)c;
                atomicOr(&a.occ_bm[p >> 5], 1u << (p & 31));
            }
        }
        __syncthreads();
        if (tid < kGR) {
            uint32_t add = 0u;
            for (int w = 0; w < kGWaves; ++w) add += s_cnt[par][w][tid];
            if (s_d[tid] > 0) s_run[tid] += add;
        }
    }
}

__global__ void __launch_bounds__(kGThreadsR) row_grad_kernel(RowGradArgs a)
{
    __shared__ RowGradLds sh;
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
        hipLaunchKernelGGL(row_grad_kernel, dim3((unsigned)blocks), dim3(kGThreadsR), 0, s, g);
        SNACK_HIP(hipGetLastError());
    }
    return SNACK_OK;
}

}  // namespace snack
