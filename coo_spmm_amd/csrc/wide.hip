// wide.hip -- the passes of wide batches (more than one 64-column batch tile)
// over views whose keys hold few entries: the 99 %-sparse layers of a
// transformer MLP at a thousand tokens, where a key's handful of entries
// gives the slice-tiled and key-major kernels too little to share per load.
//
// wide_spmm_kernel (forward over the row view, dX over the column view):
//   out[b, j] = sum over the entries e of key j of v_e * ft[idx_e, b]
// with ft the feature-major operand [nidx][bp] (zero past the batch).  A
// workgroup takes 64 batch columns (one per lane) and a block of keys, a
// wavefront a run of 1-4 consecutive keys, whose entries it streams as one
// run: the indices and values are uniform (scalar loads), every entry is one
// coalesced 256-byte row segment of ft from L2 and one fused multiply-add per
// lane, in entry order.  The key x column tile goes through LDS so that the
// batch-major stores are whole rows.
//
// wide_sddmm_kernel (dW over the canonical entries):
//   dW[e] = sum over b of dyt[r_e, b] * xt[c_e, b]
// one wavefront per entry: lane l sums the columns l, l + 64, ... in order,
// then a fixed butterfly adds the 64 lane sums.
#include "internal.h"

namespace snack {
namespace {

constexpr int kWideThreads = 256;              // the dW pass
constexpr int kWideWaves = kWideThreads / kWave;
constexpr int kWideSpmmThreads = 1024;         // the SpMM pass: 16 wavefronts, 1 to 4 keys each
constexpr int kWideSpmmWaves = kWideSpmmThreads / kWave;
constexpr int kWideU = 8;            // entries whose operand rows are loaded together
constexpr int kWideShortKey = 40;    // most entries per key (on average) for these passes

template <int R>
__global__ void __launch_bounds__(kWideSpmmThreads)
wide_spmm_kernel(const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx, const float* __restrict__ vals,
                 int32_t nkeys, const float* __restrict__ ft, int32_t bp, int32_t B, float* __restrict__ out)
{
    constexpr int KPW = R / kWideSpmmWaves;   // consecutive keys of one wavefront
    __shared__ float tile[R][kWave + 1];
    const int32_t j0 = (int32_t)blockIdx.x * R;
    const int32_t t0 = (int32_t)blockIdx.y * kWave;
    const int lane = (int)(threadIdx.x & (kWave - 1));
    // the wavefront index is uniform: said so, every key index and address below is too (scalar loads)
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const float* __restrict__ col = ft + t0 + lane;
    const int32_t jw = j0 + wv * KPW;                            // the wavefront's first key
    int kl = 0;                                                  // its key being summed
    float acc = 0.0f;
    if (jw < nkeys) {
        const int32_t jn = jw + KPW < nkeys ? jw + KPW : nkeys;
        // the keys' entries are one run: taken in groups whose loads are all issued first, a key's
        // sum going to LDS where the next key's entries begin
        const int32_t P1 = ptr[jn];
        int32_t kend = ptr[jw + 1];
        for (int32_t e0 = ptr[jw]; e0 < P1; e0 += kWideU) {
            const int32_t n = P1 - e0;
            // the arrays are padded past nnz, so the loads of a short last group stay in bounds;
            // their lanes' sums are not changed (a zero product of a non-finite operand would be NaN)
            int32_t c[kWideU];
            float v[kWideU], x[kWideU];
#pragma unroll
            for (int u = 0; u < kWideU; ++u) {
                c[u] = u < n ? idx[e0 + u] : 0;
                v[u] = vals[e0 + u];
            }
#pragma unroll
            for (int u = 0; u < kWideU; ++u) x[u] = col[(int64_t)c[u] * bp];
#pragma unroll
            for (int u = 0; u < kWideU; ++u) {
                if (u >= n) break;
                while (e0 + u >= kend) {   // the next key (empty keys pass straight through)
                    tile[wv * KPW + kl][lane] = acc;
                    acc = 0.0f;
                    ++kl;
                    kend = ptr[jw + kl + 1];
                }
                acc = fmaf(v[u], x[u], acc);
            }
        }
    }
    for (; kl < KPW; ++kl) {   // the last key summed, and keys with no entries after it
        tile[wv * KPW + kl][lane] = acc;
        acc = 0.0f;
    }
    __syncthreads();
    // the tile's rows of out: column t0 + tt, keys j0 .. j0 + R - 1
    for (int q = (int)threadIdx.x; q < kWave * R; q += kWideSpmmThreads) {
        const int tt = q / R, jj = q % R;
        const int32_t b = t0 + tt, j = j0 + jj;
        if (b < B && j < nkeys) out[(int64_t)b * nkeys + j] = tile[jj][tt];
    }
}

__global__ void __launch_bounds__(kWideThreads)
wide_sddmm_kernel(const int32_t* __restrict__ rows, const int32_t* __restrict__ cols, int64_t nnz,
                  const float* __restrict__ xt, const float* __restrict__ dyt, int32_t bp, float* __restrict__ dW)
{
    const int lane = (int)(threadIdx.x & (kWave - 1));
    const int64_t wave0 = (int64_t)blockIdx.x * kWideWaves + __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int64_t nwaves = (int64_t)gridDim.x * kWideWaves;
    for (int64_t e = wave0; e < nnz; e += nwaves) {
        const float* __restrict__ y = dyt + (int64_t)rows[e] * bp + lane;
        const float* __restrict__ x = xt + (int64_t)cols[e] * bp + lane;
        float acc = 0.0f;
        int32_t b = 0;
        for (; b + 4 * kWave <= bp; b += 4 * kWave) {
            float yy[4], xx[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                yy[u] = y[b + u * kWave];
                xx[u] = x[b + u * kWave];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) acc = fmaf(yy[u], xx[u], acc);
        }
        for (; b < bp; b += kWave) acc = fmaf(y[b], x[b], acc);
#pragma unroll
        for (int d = kWave / 2; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, kWave);
        if (lane == 0) dW[e] = acc;
    }
}

}  // namespace

bool wide_short(const snack_layer* L, const View& v, const BatchPlan& p)
{
    return p.ntiles > 1 && p.bp % kWave == 0 && L->nnz > 0 && v.nkeys > 0 &&
           L->nnz <= (int64_t)kWideShortKey * v.nkeys;
}

snack_status wide_spmm(const snack_layer* L, const View& v, const float* ft, const BatchPlan& p, int B, float* out,
                       hipStream_t s)
{
    if (!wide_short(L, v, p)) return SNACK_ERR_INVALID_ARG;
    const unsigned ty = (unsigned)(p.bp / kWave);
    // keys per workgroup: the largest of 64, 32, 16 that still gives about eight wavefronts per SIMD
    auto kblocks = [&](int R) { return (int64_t)(v.nkeys + R - 1) / R; };
    if (kblocks(64) * ty * kWideSpmmWaves >= 8192)
        hipLaunchKernelGGL(wide_spmm_kernel<64>, dim3((unsigned)kblocks(64), ty), dim3(kWideSpmmThreads), 0, s, v.ptr,
                           v.idx, v.vals, v.nkeys, ft, p.bp, B, out);
    else if (kblocks(32) * ty * kWideSpmmWaves >= 8192)
        hipLaunchKernelGGL(wide_spmm_kernel<32>, dim3((unsigned)kblocks(32), ty), dim3(kWideSpmmThreads), 0, s, v.ptr,
                           v.idx, v.vals, v.nkeys, ft, p.bp, B, out);
    else
        hipLaunchKernelGGL(wide_spmm_kernel<16>, dim3((unsigned)kblocks(16), ty), dim3(kWideSpmmThreads), 0, s, v.ptr,
                           v.idx, v.vals, v.nkeys, ft, p.bp, B, out);
    SNACK_HIP(hipGetLastError());
    return SNACK_OK;
}

snack_status wide_sddmm(const snack_layer* L, const float* xt, const float* dyt, const BatchPlan& p, float* dW,
                        hipStream_t s)
{
    if (!wide_short(L, L->fwd, p)) return SNACK_ERR_INVALID_ARG;
    int64_t blocks = (L->nnz + kWideWaves - 1) / kWideWaves;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(wide_sddmm_kernel, dim3((unsigned)blocks), dim3(kWideThreads), 0, s, L->rows, L->cols, L->nnz,
                       xt, dyt, p.bp, dW);
    SNACK_HIP(hipGetLastError());
    return SNACK_OK;
}

}  // namespace snack
