// rigl.hip -- the regrow step of a gradient-driven DST update: among the cells
// left empty by the drop, mark the `need` cells of largest |dL/dW| in the
// occupancy bitmap.  The "Padded-CSR" post (section 4.3) describes RigL as
// dropping a fraction of the live entries and growing as many "at
// high-gradient locations"; the SNACK paper (Tables 8-9) runs RigL on the
// truly sparse layer.  The gradient of the loss with respect to the dense
// weight at cell (r, c) is g = sum_b dY[b, r] X[b, c] (the dense counterpart
// of the sampled product of the backward, "Padded-CSR" section 7.1).
//
// g is accumulated in fp32 with one fused multiply-add per batch row, in batch
// order, and the decision is taken on its order key: the IEEE bits of |g| (a
// NaN counts as 0), larger first, ties by smaller linear position r*K + c.
// Nothing of size M*K is ever stored: the scores are recomputed by five sweeps
// over the cells in tiles of 128 x 128 (each thread an 8 x 8 block of fused
// multiply-add chains over batch chunks staged in LDS), which
//   1-3  histogram the order key digit by digit (bits 30-20, 19-8, 7-0) among
//        the empty cells matching the digits picked so far, a single
//        workgroup picking each digit from the top: this finds the key T of
//        the need-th best cell and how many beat it;
//   4    set every empty cell whose key beats T in the bitmap and count the
//        cells equal to T per row and column tile (in position order, so an
//        exclusive scan of the counts ranks them);
//   5    set the cells equal to T whose rank is below the remaining count.
// Every step is deterministic; bitmap words are set with atomic ORs.
#include "internal.h"

namespace snack {
namespace {

constexpr int kGT = kGradTile;          // tile rows and columns
constexpr int kGThreads = 256;          // 16 x 16 threads, 8 x 8 cells each
constexpr int kGBatch = 32;             // batch rows staged per chunk
constexpr int kH1 = 2048, kH2 = 4096, kH3 = 256;   // digit bins of passes 1-3
// state words
constexpr int kSNeed = 0;   // cells still to place (after the picks: ties to take at T)
constexpr int kST1 = 1, kST2 = 2, kST3 = 3;

enum GradMode { kHist1 = 1, kHist2 = 2, kHist3 = 3, kMark = 4, kTies = 5 };

struct GradArgs {
    const float* X;
    const float* dY;
    int32_t B, M, K;
    int32_t nct;               // column tiles
    const uint32_t* kept;
    uint32_t* occ;
    int64_t words;
    uint32_t* state;
    uint32_t* hist;
    int32_t* tie;              // counts, then their exclusive prefixes (position order)
};

__device__ inline uint32_t score_key(float g)
{
    return g != g ? 0u : (__float_as_uint(g) & 0x7FFFFFFFu);
}

// The 8 x 8 block of scores of this thread: rows r0 + ty*8 + i, columns
// c0 + tx*8 + j, each the fp32 chain acc = fma(dY[b, r], X[b, c], acc) over
// b = 0, 1, ..., B-1.
__device__ inline void tile_scores(const GradArgs& a, int r0, int c0, int ty, int tx, float (&acc)[8][8])
{
    __shared__ __align__(16) float sY[kGBatch][kGT];
    __shared__ __align__(16) float sX[kGBatch][kGT];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
    for (int b0 = 0; b0 < a.B; b0 += kGBatch) {
        const int nb = a.B - b0 < kGBatch ? a.B - b0 : kGBatch;
        __syncthreads();   // the previous chunk is consumed
        for (int q = threadIdx.x; q < kGBatch * kGT; q += kGThreads) {
            const int bb = q / kGT, j = q - bb * kGT;
            const bool inb = bb < nb;
            const int r = r0 + j, c = c0 + j;
            sY[bb][j] = (inb && r < a.M) ? a.dY[(int64_t)(b0 + bb) * a.M + r] : 0.0f;
            sX[bb][j] = (inb && c < a.K) ? a.X[(int64_t)(b0 + bb) * a.K + c] : 0.0f;
        }
        __syncthreads();
        for (int bb = 0; bb < nb; ++bb) {
            const float4 y0 = *reinterpret_cast<const float4*>(&sY[bb][ty * 8]);
            const float4 y1 = *reinterpret_cast<const float4*>(&sY[bb][ty * 8 + 4]);
            const float4 x0 = *reinterpret_cast<const float4*>(&sX[bb][tx * 8]);
            const float4 x1 = *reinterpret_cast<const float4*>(&sX[bb][tx * 8 + 4]);
            const float y[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
            const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(y[i], x[j], acc[i][j]);
        }
    }
}

// bit of cell p of a bitmap (0 past its end)
__device__ inline uint32_t bm_bits8(const uint32_t* __restrict__ bm, int64_t words, uint64_t p)
{
    // the eight cells p .. p+7: they span at most two words
    const uint64_t w = p >> 5;
    const uint32_t lo = w < (uint64_t)words ? bm[w] : 0u;
    const uint32_t hi = w + 1 < (uint64_t)words ? bm[w + 1] : 0u;
    const uint64_t both = ((uint64_t)hi << 32) | lo;
    return (uint32_t)(both >> (p & 31)) & 0xFFu;
}

template <int MODE>
__global__ void __launch_bounds__(kGThreads) grad_cells_kernel(GradArgs a)
{
    __shared__ uint32_t h[MODE == kHist1 ? kH1 : (MODE == kHist2 ? kH2 : (MODE == kHist3 ? kH3 : 1))];
    __shared__ int32_t rowcnt[kGT][16];   // ties per tile row and thread column (modes 4, 5)
    const int ct = (int)blockIdx.x, rt = (int)blockIdx.y;
    const int r0 = rt * kGT, c0 = ct * kGT;
    const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
    constexpr int NH = MODE == kHist1 ? kH1 : (MODE == kHist2 ? kH2 : (MODE == kHist3 ? kH3 : 0));
    const uint32_t t1 = a.state[kST1], t2 = a.state[kST2], t3 = a.state[kST3];
    const uint32_t T = (t1 << 20) | (t2 << 8) | t3;
    if constexpr (MODE == kTies) {
        // the smallest prefix of the tile (its first row) already reaches the ties to take: nothing here
        const int32_t need = (int32_t)a.state[kSNeed];
        if (a.tie[(int64_t)r0 * a.nct + ct] >= need) return;
    }
    for (int q = tid; q < NH; q += kGThreads) h[q] = 0u;
    if constexpr (MODE >= kMark)
        for (int q = tid; q < kGT * 16; q += kGThreads) (&rowcnt[0][0])[q] = 0;
    float acc[8][8];
    tile_scores(a, r0, c0, ty, tx, acc);   // begins and ends with a barrier around LDS use
    __syncthreads();

    // the order keys replace the scores in place (as bit patterns)
    float (&key)[8][8] = acc;
    uint32_t empty[8];   // bit j: cell (i, j) lies in the matrix and is empty after the drop
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = r0 + ty * 8 + i;
        const int cb = c0 + tx * 8;
        uint32_t m = 0u;
        if (r < a.M && cb < a.K) {
            const uint64_t p = (uint64_t)r * a.K + cb;
            m = ~bm_bits8(a.kept, a.words, p) & 0xFFu;
            const int in = a.K - cb < 8 ? a.K - cb : 8;
            m &= (1u << in) - 1u;
        }
        empty[i] = m;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = __uint_as_float(score_key(acc[i][j]));
    }

    if constexpr (MODE <= kHist3) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (!((empty[i] >> j) & 1u)) continue;
                const uint32_t k = __float_as_uint(key[i][j]);
                if (MODE == kHist1) atomicAdd(&h[k >> 20], 1u);
                else if (MODE == kHist2) { if ((k >> 20) == t1) atomicAdd(&h[(k >> 8) & 0xFFFu], 1u); }
                else { if ((k >> 8) == ((t1 << 12) | t2)) atomicAdd(&h[k & 0xFFu], 1u); }
            }
        __syncthreads();
        uint32_t* gh = a.hist + (MODE == kHist1 ? 0 : (MODE == kHist2 ? kH1 : kH1 + kH2));
        for (int q = tid; q < NH; q += kGThreads)
            if (h[q]) atomicAdd(&gh[q], h[q]);
        return;
    } else {
        // ties at T: per row, this thread's count, then (mode 5) its rank among the row's ties in the tile
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int n = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) n += (((empty[i] >> j) & 1u) && __float_as_uint(key[i][j]) == T) ? 1 : 0;
            rowcnt[ty * 8 + i][tx] = n;
        }
        __syncthreads();
        if constexpr (MODE == kMark) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = r0 + ty * 8 + i;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (!((empty[i] >> j) & 1u) || __float_as_uint(key[i][j]) <= T) continue;
                    const uint64_t p = (uint64_t)r * a.K + (c0 + tx * 8 + j);
                    atomicOr(&a.occ[p >> 5], 1u << (p & 31));
                }
            }
            if (tid < kGT && r0 + tid < a.M) {
                int32_t n = 0;
                for (int t = 0; t < 16; ++t) n += rowcnt[tid][t];
                a.tie[(int64_t)(r0 + tid) * a.nct + ct] = n;
            }
        } else {
            const int32_t need = (int32_t)a.state[kSNeed];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int rl = ty * 8 + i;
                const int r = r0 + rl;
                if (r >= a.M) continue;
                int32_t rank = a.tie[(int64_t)r * a.nct + ct];
                for (int t = 0; t < tx; ++t) rank += rowcnt[rl][t];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (!((empty[i] >> j) & 1u) || __float_as_uint(key[i][j]) != T) continue;
                    if (rank < need) {
                        const uint64_t p = (uint64_t)r * a.K + (c0 + tx * 8 + j);
                        atomicOr(&a.occ[p >> 5], 1u << (p & 31));
                    }
                    ++rank;
                }
            }
        }
    }
}

// state: need, and the histograms cleared
__global__ void grad_init_kernel(uint32_t* __restrict__ state, uint32_t* __restrict__ hist, uint32_t need)
{
    for (int q = threadIdx.x; q < kGradHistWords; q += blockDim.x) hist[q] = 0u;
    if (threadIdx.x < 16) state[threadIdx.x] = threadIdx.x == kSNeed ? need : 0u;
}

// occ = kept
__global__ void grad_copy_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst, int64_t words)
{
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < words; q += (int64_t)gridDim.x * blockDim.x)
        dst[q] = src[q];
}

// the digit of pass `pass` that holds the need-th best key, counting from the
// largest digit down; need becomes the rank within that digit.  One
// workgroup: each thread four consecutive bins from the top, a scan of their
// sums finds the first digit (from the top, above 0) where the count reaches
// need; digit 0 takes what is left when none does.
constexpr int kPickThreads = 1024;
static_assert(kH2 <= 4 * kPickThreads, "four bins per thread");

__global__ void __launch_bounds__(kPickThreads) grad_pick_kernel(uint32_t* __restrict__ state,
                                                                 const uint32_t* __restrict__ hist, int pass)
{
    __shared__ uint32_t wsum[kPickThreads / kWave];
    __shared__ uint32_t s_found, s_t, s_rest;
    const int nb = pass == 1 ? kH1 : (pass == 2 ? kH2 : kH3);
    const uint32_t* h = hist + (pass == 1 ? 0 : (pass == 2 ? kH1 : kH1 + kH2));
    const uint32_t need = state[kSNeed];
    const int tid = (int)threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
    uint32_t c[4];
    int t[4];
    uint32_t sum = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        t[j] = nb - 1 - (4 * tid + j);
        c[j] = t[j] >= 1 ? h[t[j]] : 0u;
        sum += c[j];
    }
    uint32_t inc = sum;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const uint32_t o = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += o;
    }
    if (lane == kWave - 1) wsum[w] = inc;
    if (tid == 0) s_found = 0u;
    __syncthreads();
    uint32_t base = 0u, total = 0u;
    for (int i = 0; i < kPickThreads / kWave; ++i) {
        if (i < w) base += wsum[i];
        total += wsum[i];
    }
    inc += base;
    const uint32_t excl = inc - sum;
    if (excl < need && inc >= need) {   // exactly one thread
        uint32_t r = need - excl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (c[j] >= r) {
                s_t = (uint32_t)t[j];
                s_rest = r;
                break;
            }
            r -= c[j];
        }
        s_found = 1u;
    }
    __syncthreads();
    if (tid == 0) {
        const uint32_t tt = s_found ? s_t : 0u;
        const uint32_t rest = s_found ? s_rest : need - total;
        state[pass == 1 ? kST1 : (pass == 2 ? kST2 : kST3)] = tt;
        state[kSNeed] = rest;
    }
}

}  // namespace

snack_status grow_by_gradient(const snack_layer* L, const GradGrow& g, hipStream_t s)
{
    if (g.need <= 0) return SNACK_OK;
    if (!g.X || !g.dY || g.B < 1 || g.need > 0xFFFFFFFFll) return SNACK_ERR_INVALID_ARG;
    GradArgs a;
    a.X = g.X;
    a.dY = g.dY;
    a.B = g.B;
    a.M = L->M;
    a.K = L->K;
    a.nct = (int32_t)grad_col_tiles(L->K);
    a.kept = g.kept_bm;
    a.occ = g.occ_bm;
    a.words = g.words;
    a.state = g.state;
    a.hist = g.hist;
    a.tie = g.tie_cnt;
    const dim3 grid((unsigned)a.nct, (unsigned)((L->M + kGT - 1) / kGT)), block(kGThreads);
    hipLaunchKernelGGL(grad_init_kernel, dim3(1), dim3(256), 0, s, g.state, g.hist, (uint32_t)g.need);
    {
        int64_t nb = (g.words + 255) / 256;
        if (nb > 4096) nb = 4096;
        hipLaunchKernelGGL(grad_copy_kernel, dim3((unsigned)nb), dim3(256), 0, s, g.kept_bm, g.occ_bm, g.words);
    }
    hipLaunchKernelGGL(grad_cells_kernel<kHist1>, grid, block, 0, s, a);
    hipLaunchKernelGGL(grad_pick_kernel, dim3(1), dim3(kPickThreads), 0, s, g.state, g.hist, 1);
    hipLaunchKernelGGL(grad_cells_kernel<kHist2>, grid, block, 0, s, a);
    hipLaunchKernelGGL(grad_pick_kernel, dim3(1), dim3(kPickThreads), 0, s, g.state, g.hist, 2);
    hipLaunchKernelGGL(grad_cells_kernel<kHist3>, grid, block, 0, s, a);
    hipLaunchKernelGGL(grad_pick_kernel, dim3(1), dim3(kPickThreads), 0, s, g.state, g.hist, 3);
    hipLaunchKernelGGL(grad_cells_kernel<kMark>, grid, block, 0, s, a);
    SNACK_HIP(hipGetLastError());
    SNACK_CHECK(exclusive_scan_i32(g.tie_cnt, g.tie_cnt, (int64_t)L->M * a.nct, nullptr, g.scan, s));
    hipLaunchKernelGGL(grad_cells_kernel<kTies>, grid, block, 0, s, a);
    SNACK_HIP(hipGetLastError());
    return SNACK_OK;
}

}  // namespace snack
