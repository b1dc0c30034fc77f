// aux.hip -- feature-major activation copies and the elementwise training
// helpers (SGD, MSE gradient, exact GELU).  None of these is the sparse
// method; they keep the training loop on the device.
#include "internal.h"

#include <math.h>

namespace snack {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;

inline unsigned grid_for(int64_t n)
{
    int64_t g = (n + kThreads - 1) / kThreads;
    if (g < 1) g = 1;
    if (g > 65535LL * 8) g = 65535LL * 8;
    return (unsigned)g;
}

// dst[c * bp + b] = (b < B) ? src[b * n + c] : 0 ; one 64 x 64 tile per block via LDS.
// Blocks [0, nx1) handle (src, dst, n), the rest (src2, dst2, n2).
__global__ void __launch_bounds__(kThreads) transpose_pad_kernel(const float* __restrict__ src1,
                                                                 float* __restrict__ dst1, int n1,
                                                                 const float* __restrict__ src2,
                                                                 float* __restrict__ dst2, int n2, int nx1, int B,
                                                                 int bp)
{
    __shared__ float tile[kTile][kTile + 1];
    const bool first = (int)blockIdx.x < nx1;
    const float* __restrict__ src = first ? src1 : src2;
    float* __restrict__ dst = first ? dst1 : dst2;
    const int n = first ? n1 : n2;
    const int c0 = (first ? (int)blockIdx.x : (int)blockIdx.x - nx1) * kTile;
    const int b0 = blockIdx.y * kTile;
    const int tx = threadIdx.x & (kTile - 1);
    const int ty = threadIdx.x / kTile;   // 0..3
    for (int bb = ty; bb < kTile; bb += kThreads / kTile) {
        const int b = b0 + bb, c = c0 + tx;
        float v = 0.0f;
        if (b < B && c < n) v = src[(int64_t)b * n + c];
        tile[bb][tx] = v;
    }
    __syncthreads();
    for (int cc = ty; cc < kTile; cc += kThreads / kTile) {
        const int c = c0 + cc, b = b0 + tx;
        if (c < n && b < bp) dst[(int64_t)c * bp + b] = tile[tx][cc];
    }
}

__global__ void sgd_kernel(float* __restrict__ v, const float* __restrict__ g, float lr, int64_t n, int vec)
{
    const int64_t n4 = vec ? n / 4 : 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
        float4 a = reinterpret_cast<float4*>(v)[i];
        const float4 d = reinterpret_cast<const float4*>(g)[i];
        a.x = sgd_value(a.x, d.x, lr); a.y = sgd_value(a.y, d.y, lr); a.z = sgd_value(a.z, d.z, lr); a.w = sgd_value(a.w, d.w, lr);
        reinterpret_cast<float4*>(v)[i] = a;
    }
    for (int64_t i = n4 * 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        v[i] = sgd_value(v[i], g[i], lr);
}

// both value copies in one launch: (v, g) and (v2, g2), each n long
__global__ void sgd2_kernel(float* __restrict__ v, const float* __restrict__ g, float* __restrict__ v2,
                            const float* __restrict__ g2, float lr, int64_t n)
{
    const int64_t n4 = n / 4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 2 * n4; i += (int64_t)gridDim.x * blockDim.x) {
        const bool second = i >= n4;
        const int64_t j = second ? i - n4 : i;
        float4* __restrict__ pv = reinterpret_cast<float4*>(second ? v2 : v);
        const float4* __restrict__ pg = reinterpret_cast<const float4*>(second ? g2 : g);
        float4 a = pv[j];
        const float4 d = pg[j];
        a.x = sgd_value(a.x, d.x, lr); a.y = sgd_value(a.y, d.y, lr); a.z = sgd_value(a.z, d.z, lr); a.w = sgd_value(a.w, d.w, lr);
        pv[j] = a;
    }
    for (int64_t i = n4 * 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        v[i] = sgd_value(v[i], g[i], lr);
        v2[i] = sgd_value(v2[i], g2[i], lr);
    }
}

__global__ void mse_grad_kernel(const float* __restrict__ Y, const float* __restrict__ T, float* __restrict__ dY,
                                int64_t n, float scale)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        dY[i] = scale * (Y[i] - T[i]);
}

__global__ void gelu_fwd_kernel(const float* __restrict__ X, float* __restrict__ Y, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        Y[i] = gelu_value(X[i]);
    }
}

__global__ void gelu_bwd_kernel(const float* __restrict__ X, const float* __restrict__ dY, float* __restrict__ dX,
                                int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const float x = X[i];
        const float cdf = 0.5f * (1.0f + erff(x * 0.70710678118654752f));
        const float pdf = 0.39894228040143268f * expf(-0.5f * x * x);
        dX[i] = dY[i] * (cdf + x * pdf);
    }
}

// round to nearest even: add 0x7FFF plus the kept word's lowest bit, keep the
// high half; NaN stays a quiet NaN of the same sign
__global__ void pack_bf16_kernel(const float* __restrict__ v, uint16_t* __restrict__ o, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t b = __float_as_uint(v[i]);
        uint16_t h;
        if ((b & 0x7FFFFFFFu) > 0x7F800000u) h = (uint16_t)((b >> 16) | 0x0040u);
        else h = (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
        o[i] = h;
    }
}

}  // namespace

// Flat variant: one thread per 4 consecutive padded batch columns of one
// feature (bp a multiple of 4): four strided reads, one 16-byte store.  Many
// small workgroups instead of one 64x64 tile per workgroup.
namespace {
__global__ void __launch_bounds__(kThreads) transpose_pad4_kernel(const float* __restrict__ src1,
                                                                  float* __restrict__ dst1, int n1,
                                                                  const float* __restrict__ src2,
                                                                  float* __restrict__ dst2, int n2, int B, int bp)
{
    const int q = bp / 4;
    const int64_t total1 = (int64_t)n1 * q, total = total1 + (int64_t)n2 * q;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const bool first = i < total1;
        const int64_t j = first ? i : i - total1;
        const float* __restrict__ src = first ? src1 : src2;
        float* __restrict__ dst = first ? dst1 : dst2;
        const int n = first ? n1 : n2;
        const int c = (int)(j / q);
        const int b = (int)(j - (int64_t)c * q) * 4;
        float4 v;
        v.x = b < B ? src[(int64_t)b * n + c] : 0.0f;
        v.y = b + 1 < B ? src[(int64_t)(b + 1) * n + c] : 0.0f;
        v.z = b + 2 < B ? src[(int64_t)(b + 2) * n + c] : 0.0f;
        v.w = b + 3 < B ? src[(int64_t)(b + 3) * n + c] : 0.0f;
        *reinterpret_cast<float4*>(dst + (int64_t)c * bp + b) = v;
    }
}
// Wide batches: one 64-feature x 64-column tile per workgroup, read as 16-byte
// pieces of batch rows (16 threads per 256-byte row), transposed through LDS
// (rows padded to 65 floats, so the column reads hit distinct banks) and
// written as 16-byte pieces of feature rows.  Needs n % 4 == 0, bp % 64 == 0
// and 16-byte aligned arrays.  Blocks x in [0, nx1) handle (src, dst, n).
// (Narrow batches: the flat variant below issues one 16-byte store per
// thread and launches many more workgroups.)
__global__ void __launch_bounds__(kThreads) transpose_tile4_kernel(const float* __restrict__ src1,
                                                                   float* __restrict__ dst1, int n1,
                                                                   const float* __restrict__ src2,
                                                                   float* __restrict__ dst2, int n2, int nx1, int B,
                                                                   int bp)
{
    __shared__ float tile[kTile][kTile + 1];
    const bool first = (int)blockIdx.x < nx1;
    const float* __restrict__ src = first ? src1 : src2;
    float* __restrict__ dst = first ? dst1 : dst2;
    const int n = first ? n1 : n2;
    const int c0 = (first ? (int)blockIdx.x : (int)blockIdx.x - nx1) * kTile;
    const int b0 = (int)blockIdx.y * kTile;
    const int q = (int)threadIdx.x & 15, r = (int)threadIdx.x >> 4;   // 16-byte piece, row within a group of 16
#pragma unroll
    for (int i = 0; i < kTile / 16; ++i) {
        const int bb = r + 16 * i, b = b0 + bb, c = c0 + 4 * q;
        float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (b < B && c < n) v = *reinterpret_cast<const float4*>(src + (int64_t)b * n + c);
        tile[bb][4 * q + 0] = v.x;
        tile[bb][4 * q + 1] = v.y;
        tile[bb][4 * q + 2] = v.z;
        tile[bb][4 * q + 3] = v.w;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kTile / 16; ++i) {
        const int cc = r + 16 * i, c = c0 + cc;
        if (c < n)
            *reinterpret_cast<float4*>(dst + (int64_t)c * bp + b0 + 4 * q) =
                make_float4(tile[4 * q + 0][cc], tile[4 * q + 1][cc], tile[4 * q + 2][cc], tile[4 * q + 3][cc]);
    }
}

}  // namespace

snack_status transpose_pad(const float* src, float* dst, int n, const float* src2, float* dst2, int n2, int B,
                           int bp, hipStream_t s)
{
    ProfScope prof(KC_TRANSPOSE, s);
    const bool a16 = ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) |
                       reinterpret_cast<uintptr_t>(src2) | reinterpret_cast<uintptr_t>(dst2)) & 15) == 0;
    // from two tiles of columns on (with one, the grid is too small to beat the flat variant)
    if (bp % kTile == 0 && bp >= 2 * kTile && n % 4 == 0 && (!src2 || n2 % 4 == 0) && a16) {
        const int nx1 = (n + kTile - 1) / kTile;
        const int nx2 = src2 ? (n2 + kTile - 1) / kTile : 0;
        hipLaunchKernelGGL(transpose_tile4_kernel, dim3((unsigned)(nx1 + nx2), (unsigned)(bp / kTile)),
                           dim3(kThreads), 0, s, src, dst, n, src2, dst2, n2, nx1, B, bp);
        SNACK_HIP(hipGetLastError());
        return SNACK_OK;
    }
    if (bp % 4 == 0) {
        const int64_t total = ((int64_t)n + (src2 ? n2 : 0)) * (bp / 4);
        hipLaunchKernelGGL(transpose_pad4_kernel, dim3(grid_for(total)), dim3(kThreads), 0, s, src, dst, n, src2, dst2,
                           src2 ? n2 : 0, B, bp);
        SNACK_HIP(hipGetLastError());
        return SNACK_OK;
    }
    const int nx1 = (n + kTile - 1) / kTile;
    const int nx2 = src2 ? (n2 + kTile - 1) / kTile : 0;
    dim3 grid((unsigned)(nx1 + nx2), (unsigned)((bp + kTile - 1) / kTile));
    hipLaunchKernelGGL(transpose_pad_kernel, grid, dim3(kThreads), 0, s, src, dst, n, src2, dst2, n2, nx1, B, bp);
    SNACK_HIP(hipGetLastError());
    return SNACK_OK;
}

snack_status sgd_update(snack_layer* L, const float* dW, const float* dW_t, float lr, hipStream_t s)
{
    if (L->nnz == 0) return SNACK_OK;
    ProfScope prof(KC_SGD, s);
    const bool aligned = (((uintptr_t)dW | (uintptr_t)dW_t) & 15) == 0;
    if (dW_t && aligned) {
        unsigned g = grid_for(L->nnz / 2 + 1);
        hipLaunchKernelGGL(sgd2_kernel, dim3(g), dim3(kThreads), 0, s, L->vals, dW, L->vals_t, dW_t, lr, L->nnz);
    } else {
        hipLaunchKernelGGL(sgd_kernel, dim3(grid_for(L->nnz / 4 + 1)), dim3(kThreads), 0, s, L->vals, dW, lr,
                           L->nnz, aligned ? 1 : 0);
        if (dW_t) {
            hipLaunchKernelGGL(sgd_kernel, dim3(grid_for(L->nnz / 4 + 1)), dim3(kThreads), 0, s, L->vals_t, dW_t, lr,
                               L->nnz, 1);
        } else {
            L->vals_t_stale = true;
        }
    }
    SNACK_HIP(hipGetLastError());
    return SNACK_OK;
}

snack_status sgd_update_values(snack_layer* L, const float* dW, float lr, hipStream_t s)
{
    if (L->nnz == 0) return SNACK_OK;
    ProfScope prof(KC_SGD, s);
    const bool aligned = ((uintptr_t)dW & 15) == 0;
    hipLaunchKernelGGL(sgd_kernel, dim3(grid_for(L->nnz / 4 + 1)), dim3(kThreads), 0, s, L->vals, dW, lr, L->nnz,
                       aligned ? 1 : 0);
    SNACK_HIP(hipGetLastError());
    return SNACK_OK;
}

snack_status mse_grad(const float* Y, const float* T, float* dY, int64_t n, float scale, hipStream_t s)
{
    if (n == 0) return SNACK_OK;
    ProfScope prof(KC_ELEMENTWISE, s);
    hipLaunchKernelGGL(mse_grad_kernel, dim3(grid_for(n)), dim3(kThreads), 0, s, Y, T, dY, n, scale);
    SNACK_HIP(hipGetLastError());
    return SNACK_OK;
}

snack_status gelu_fwd(const float* X, float* Y, int64_t n, hipStream_t s)
{
    if (n == 0) return SNACK_OK;
    ProfScope prof(KC_ELEMENTWISE, s);
    hipLaunchKernelGGL(gelu_fwd_kernel, dim3(grid_for(n)), dim3(kThreads), 0, s, X, Y, n);
    SNACK_HIP(hipGetLastError());
    return SNACK_OK;
}

snack_status pack_bf16(snack_layer* L, hipStream_t s)
{
    if (!L->vals16) return SNACK_ERR_UNSUPPORTED;
    if (L->nnz > 0) {
        ProfScope prof(KC_ELEMENTWISE, s);
        hipLaunchKernelGGL(pack_bf16_kernel, dim3(grid_for(L->nnz)), dim3(kThreads), 0, s, L->vals, L->vals16, L->nnz);
        SNACK_HIP(hipGetLastError());
    }
    L->b16_version = L->vals_version;
    return SNACK_OK;
}

snack_status gelu_bwd(const float* X, const float* dY, float* dX, int64_t n, hipStream_t s)
{
    if (n == 0) return SNACK_OK;
    ProfScope prof(KC_ELEMENTWISE, s);
    hipLaunchKernelGGL(gelu_bwd_kernel, dim3(grid_for(n)), dim3(kThreads), 0, s, X, dY, dX, n);
    SNACK_HIP(hipGetLastError());
    return SNACK_OK;
}

}  // namespace snack
