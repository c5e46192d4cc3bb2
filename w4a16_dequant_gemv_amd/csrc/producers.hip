// producers.hip -- GPTQ and AWQ: calibration-driven producers of the packed
// group-wise weight format that q4_quantize_pack writes.
//
// GPTQ ([Guide] §4.3): minimize ||X W^T - X W_hat^T|| layer by layer.  H =
// 2 X^T X from calibration tokens, damped by lambda * mean(diag H); U, the
// upper Cholesky factor of H^-1; then column by column, the group's scale and
// zero-point from the current (already compensated) weights, the column's
// code, and its error (w - w') / U[i][i] pushed onto every later column as
// w_j -= err * U[i][j], applied lazily in blocks of 128 columns.
// AWQ ([Guide] §4.4): per input channel s_j = (mean |X_j|)^alpha, weights
// scaled by s before group-wise quantization and activations divided by s,
// alpha searched on a grid over [0, 1] for the smallest output error on the
// calibration tokens.
//
// Everything is arranged so that each value is produced by the same sequence
// of IEEE operations as in a plain sequential implementation of the pages'
// loops (this unit is built without FMA contraction and with correctly
// rounded division and square root):
//   * H: one binary64 sum per element over the tokens in order, written
//     straight into the index-reversed layout the factorization wants;
//   * U = J L^-1 J with J H J = L L^T: a right-looking Cholesky and a
//     right-looking triangular inverse in binary64, one launch per pivot and
//     step, every element receiving its updates in pivot order (L is kept
//     transposed so that a pivot's column is a contiguous row);
//   * the column loop in binary32: each 128-column block is processed one
//     column after another per row with the block's weights in LDS, and the
//     block's errors then reach the later columns in column order, so lazy
//     updates give the same values as immediate ones;
//   * AWQ's losses: each output error sums over k in order in binary64, then
//     over tokens, then over output channels, in order.
#include <mutex>

#include "q4_device.h"
#include "q4_launch.h"

namespace {

constexpr int kThreads = 256;
constexpr int kBlock = 128;              // GPTQ lazy-update block (columns)

// ---------------------------------------------------------------------------
// GPTQ: Hessian, damping, factor.
// ---------------------------------------------------------------------------

// 32 x 32 tile (ti, tj), ti >= tj, of H = 2 X^T X; element (i, j), i >= j, is
// stored at S[n-1-i][n-1-j] (the upper triangle of J H J).
__global__ __launch_bounds__(kThreads) void hessian_kernel(const uint16_t *__restrict__ x, int64_t t, int n,
                                                           double *__restrict__ S)
{
    __shared__ double xa[64][33], xb[64][33];
    // lower-triangular tile index -> (ti, tj)
    const int64_t b = blockIdx.x;
    int ti = (int)((sqrt(8.0 * (double)b + 1.0) - 1.0) / 2.0);
    while ((int64_t)(ti + 1) * (ti + 2) / 2 <= b) ++ti;
    while ((int64_t)ti * (ti + 1) / 2 > b) --ti;
    const int tj = (int)(b - (int64_t)ti * (ti + 1) / 2);
    const int i0 = ti * 32, j0 = tj * 32;
    const int row = threadIdx.x / 8, col = (threadIdx.x % 8) * 4;
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for (int64_t t0 = 0; t0 < t; t0 += 64) {
        for (int e = threadIdx.x; e < 64 * 32; e += kThreads) {
            const int rr = e / 32, cc = e % 32;
            const int64_t tt = t0 + rr;
            double va = 0.0, vb = 0.0;
            if (tt < t) {
                if (i0 + cc < n) va = (double)half_bits_to_float(x[tt * n + i0 + cc]);
                if (j0 + cc < n) vb = (double)half_bits_to_float(x[tt * n + j0 + cc]);
            }
            xa[rr][cc] = va;
            xb[rr][cc] = vb;
        }
        __syncthreads();
        const int steps = (int)(t - t0 < 64 ? t - t0 : 64);
        for (int rr = 0; rr < steps; ++rr) {
            const double a = xa[rr][row];
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = acc[c] + a * xb[rr][col + c];
        }
        __syncthreads();
    }
    const int i = i0 + row;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int j = j0 + col + c;
        if (i < n && j <= i) S[(int64_t)(n - 1 - i) * n + (n - 1 - j)] = 2.0 * acc[c];
    }
}

// Adds lambda * mean(diag H) to the diagonal; the diagonal is summed in the
// original index order.
__global__ __launch_bounds__(kThreads) void damp_kernel(double *__restrict__ S, int n, double lambda)
{
    __shared__ double add;
    if (threadIdx.x == 0) {
        double sum = 0.0;
        for (int i = 0; i < n; ++i) sum += S[(int64_t)(n - 1 - i) * n + (n - 1 - i)];
        add = lambda * (sum / (double)n);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kThreads) S[(int64_t)i * n + i] += add;
}

// Cholesky pivot j, step 1: l[i][j] = a[i][j] / sqrt(a[j][j]) for i > j (row
// j of S).  The diagonal itself is replaced in step 2, which does not read it,
// so no workgroup here can see it changed.
__global__ __launch_bounds__(kThreads) void chol_scale_kernel(double *__restrict__ S, int n, int j)
{
    const double d = sqrt(S[(int64_t)j * n + j]);
    const int i = j + 1 + blockIdx.x * kThreads + threadIdx.x;
    if (i < n) S[(int64_t)j * n + i] = S[(int64_t)j * n + i] / d;
}

// Cholesky pivot j, step 2: l[j][j] = sqrt(a[j][j]), and a[i][k] -= l[i][j] *
// l[k][j] for j < k <= i (row k of S, columns i >= k).  Launched with at least
// one row of blocks so the diagonal is written for the last pivot too.
__global__ __launch_bounds__(kThreads) void chol_update_kernel(double *__restrict__ S, int n, int j)
{
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
        S[(int64_t)j * n + j] = sqrt(S[(int64_t)j * n + j]);
    const int k = j + 1 + blockIdx.y;
    if (k >= n) return;
    const int i = k + blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    const double ljk = S[(int64_t)j * n + k];
    S[(int64_t)k * n + i] = S[(int64_t)k * n + i] - S[(int64_t)j * n + i] * ljk;
}

__global__ __launch_bounds__(kThreads) void identity_kernel(double *__restrict__ M, int n)
{
    const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (e < (int64_t)n * n) M[e] = (e / n == e % n) ? 1.0 : 0.0;
}

// Triangular inverse pivot j, step 1: row j of M divided by l[j][j].
__global__ __launch_bounds__(kThreads) void inv_scale_kernel(const double *__restrict__ S, double *__restrict__ M,
                                                             int n, int j)
{
    const int c = blockIdx.x * kThreads + threadIdx.x;
    if (c <= j) M[(int64_t)j * n + c] = M[(int64_t)j * n + c] / S[(int64_t)j * n + j];
}

// Triangular inverse pivot j, step 2: m[i][c] -= l[i][j] * m[j][c] for i > j, c <= j.
__global__ __launch_bounds__(kThreads) void inv_update_kernel(const double *__restrict__ S, double *__restrict__ M,
                                                              int n, int j)
{
    const int i = j + 1 + blockIdx.y;
    const int c = blockIdx.x * kThreads + threadIdx.x;
    if (c > j) return;
    const double lij = S[(int64_t)j * n + i];
    M[(int64_t)i * n + c] = M[(int64_t)i * n + c] - lij * M[(int64_t)j * n + c];
}

// U[a][b] = fp32(M[n-1-a][n-1-b]) for a <= b, zero below the diagonal.
__global__ __launch_bounds__(kThreads) void u_from_inverse_kernel(const double *__restrict__ M, int n,
                                                                  float *__restrict__ U)
{
    const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (e >= (int64_t)n * n) return;
    const int a = (int)(e / n), b = (int)(e % n);
    U[e] = a <= b ? (float)M[(int64_t)(n - 1 - a) * n + (n - 1 - b)] : 0.0f;
}

// ---------------------------------------------------------------------------
// GPTQ: the column loop.
// ---------------------------------------------------------------------------
template <int BITS, bool SYM>
struct GroupMap {
    static constexpr float TOP = SYM ? (float)((1 << (BITS - 1)) - 1) : (float)((1 << BITS) - 1);
    static constexpr float BOTTOM = SYM ? -(float)(1 << (BITS - 1)) : 0.0f;
    static constexpr int OFFSET = 1 << (BITS - 1);
};

// One thread per row: columns [b0, b1) one after another with the block in
// LDS, errors to E[row][0 .. b1-b0).  The row's current fp32 scale and
// zero-point live in SZ[row] across blocks (a group of 256 columns, or a
// whole row, spans several blocks).
template <int BITS, bool SYM>
__global__ __launch_bounds__(64) void gptq_block_kernel(const float *__restrict__ W, const float *__restrict__ U,
                                                       int64_t n_out, int n, int b0, int b1, int group_size,
                                                       float *__restrict__ E, float *__restrict__ SZ,
                                                       uint32_t *__restrict__ qweight,
                                                       uint16_t *__restrict__ scales, uint16_t *__restrict__ zeros)
{
    using G = GroupMap<BITS, SYM>;
    constexpr int PER_WORD = 32 / BITS;
    // dynamic LDS: the block's weights [kBlock][64] and its U block [kBlock][kBlock + 1]
    extern __shared__ float dyn_lds[];
    float (*wblk)[64] = reinterpret_cast<float (*)[64]>(dyn_lds);
    float (*ublk)[kBlock + 1] = reinterpret_cast<float (*)[kBlock + 1]>(dyn_lds + kBlock * 64);
    const int tid = threadIdx.x;
    const int64_t row = (int64_t)blockIdx.x * 64 + tid;
    const int width = b1 - b0;
    for (int e = tid; e < width * width; e += 64) {
        const int a = e / width, c = e % width;
        ublk[a][c] = U[(int64_t)(b0 + a) * n + b0 + c];
    }
    const bool live = row < n_out;
    const int64_t rr = live ? row : n_out - 1;
    for (int c = 0; c < width; ++c) wblk[c][tid] = W[rr * n + b0 + c];
    __syncthreads();
    if (!live) return;
    const int groups = n / group_size;
    float s = SZ[2 * row], z = SZ[2 * row + 1];                  // the open group's, if b0 is inside one
    float s16 = (float)(_Float16)s;
    uint32_t word = 0;
    for (int i = b0; i < b1; ++i) {
        const int li = i - b0;
        if (i % group_size == 0) {
            float lo = 0.0f, hi = 0.0f;
            for (int c = i; c < i + group_size; ++c) {
                const float v = c < b1 ? wblk[c - b0][tid] : W[rr * n + c];
                if (c == i) {
                    lo = hi = SYM ? fabsf(v) : v;
                } else if (SYM) {
                    hi = fmaxf(hi, fabsf(v));
                } else {
                    lo = fminf(lo, v);
                    hi = fmaxf(hi, v);
                }
            }
            if (SYM) {
                s = hi / G::TOP;
                if (s < 1e-8f) s = 1e-8f;
                z = 0.0f;
            } else {
                s = (hi - lo) / G::TOP;
                if (s < 1e-8f) s = 1e-8f;
                z = fminf(fmaxf(__builtin_rintf(-lo / s), 0.0f), G::TOP);
            }
            const _Float16 sh = (_Float16)s;
            s16 = (float)sh;
            SZ[2 * row] = s;
            SZ[2 * row + 1] = z;
            scales[row * groups + i / group_size] = bitcast<uint16_t>(sh);
            zeros[row * groups + i / group_size] = bitcast<uint16_t>((_Float16)(SYM ? (float)G::OFFSET : z));
        }
        const float w = wblk[li][tid];
        const float q = fminf(fmaxf(__builtin_rintf(w / s) + z, G::BOTTOM), G::TOP);
        const float deq = s16 * (q - z);
        const float err = (w - deq) / ublk[li][li];
        const uint32_t code = (uint32_t)(int32_t)(SYM ? q + (float)G::OFFSET : q);
        word |= code << (BITS * (i % PER_WORD));
        if (i % PER_WORD == PER_WORD - 1) {
            qweight[row * (n / PER_WORD) + i / PER_WORD] = word;
            word = 0;
        }
        for (int c = li + 1; c < width; ++c) wblk[c][tid] = wblk[c][tid] - err * ublk[li][c];
        E[row * kBlock + li] = err;
    }
}

// Later columns j >= b1 of every row: w -= E[row][i - b0] * U[i][j] for i in
// [b0, b1) in order.  64 x 32 tiles, 2 x 4 elements per thread.
__global__ __launch_bounds__(kThreads) void gptq_trailing_kernel(float *__restrict__ W, const float *__restrict__ U,
                                                                 const float *__restrict__ E, int64_t n_out, int n,
                                                                 int b0, int b1)
{
    __shared__ float e_lds[64][kBlock + 1];
    __shared__ float u_lds[kBlock][32];
    const int width = b1 - b0;
    const int64_t r0 = (int64_t)blockIdx.x * 64;
    const int c0 = b1 + blockIdx.y * 32;
    for (int e = threadIdx.x; e < 64 * width; e += kThreads) {
        const int rr = e / width, ii = e % width;
        e_lds[rr][ii] = r0 + rr < n_out ? E[(r0 + rr) * kBlock + ii] : 0.0f;
    }
    for (int e = threadIdx.x; e < width * 32; e += kThreads) {
        const int ii = e / 32, cc = e % 32;
        u_lds[ii][cc] = c0 + cc < n ? U[(int64_t)(b0 + ii) * n + c0 + cc] : 0.0f;
    }
    __syncthreads();
    const int tr = (threadIdx.x / 8) * 2, tc = (threadIdx.x % 8) * 4;
    float v[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t r = r0 + tr + a;
            const int c = c0 + tc + b;
            v[a][b] = (r < n_out && c < n) ? W[r * n + c] : 0.0f;
        }
    for (int ii = 0; ii < width; ++ii) {
#pragma unroll
        for (int a = 0; a < 2; ++a) {
            const float e = e_lds[tr + a][ii];
#pragma unroll
            for (int b = 0; b < 4; ++b) v[a][b] = v[a][b] - e * u_lds[ii][tc + b];
        }
    }
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int64_t r = r0 + tr + a;
            const int c = c0 + tc + b;
            if (r < n_out && c < n) W[r * n + c] = v[a][b];
        }
}

// ---------------------------------------------------------------------------
// AWQ.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void act_mean_kernel(const uint16_t *__restrict__ x, int64_t t, int n,
                                                            double *__restrict__ mean)
{
    const int j = blockIdx.x * kThreads + threadIdx.x;
    if (j >= n) return;
    double acc = 0.0;
    for (int64_t r = 0; r < t; ++r) acc += fabs((double)half_bits_to_float(x[r * n + j]));
    mean[j] = acc / (double)t;
}

// s = max(float(pow(mean, alpha)), 1e-5) with alpha = index / n_grid; index
// from *best when best is given (the search's winner).
__global__ __launch_bounds__(kThreads) void awq_scales_kernel(const double *__restrict__ mean, int n, int index,
                                                              int n_grid, const int32_t *__restrict__ best,
                                                              float *__restrict__ s)
{
    const int j = blockIdx.x * kThreads + threadIdx.x;
    if (j >= n) return;
    const int idx = best ? *best : index;
    const double alpha = (double)idx / (double)n_grid;
    const float v = (float)pow(mean[j], alpha);
    s[j] = v < 1e-5f ? 1e-5f : v;
}

__global__ __launch_bounds__(kThreads) void scale_columns_kernel(const float *__restrict__ w, const float *__restrict__ s,
                                                                 int64_t total, int n, float *__restrict__ out)
{
    const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (e < total) out[e] = w[e] * s[e % n];
}

// y[c][r] = sum_k x[r][k] * (w[c][k] - deq[c][k] / s[k]) in binary64, k in
// order; 16 x 16 (token, channel) tiles with k staged through LDS.
__global__ __launch_bounds__(kThreads) void awq_out_err_kernel(const uint16_t *__restrict__ x, const float *__restrict__ w,
                                                               const float *__restrict__ deq, const float *__restrict__ s,
                                                               int64_t t, int64_t n_out, int n, double *__restrict__ y)
{
    __shared__ double xs[16][65], ds[16][65];
    const int64_t r0 = (int64_t)blockIdx.x * 16, c0 = (int64_t)blockIdx.y * 16;
    const int tr = threadIdx.x / 16, tc = threadIdx.x % 16;
    double acc = 0.0;
    for (int k0 = 0; k0 < n; k0 += 64) {
        for (int e = threadIdx.x; e < 16 * 64; e += kThreads) {
            const int a = e / 64, kk = e % 64, k = k0 + kk;
            const int64_t r = r0 + a, c = c0 + a;
            xs[a][kk] = (r < t && k < n) ? (double)half_bits_to_float(x[r * n + k]) : 0.0;
            double d = 0.0;
            if (c < n_out && k < n) {
                const float weff = deq[c * n + k] / s[k];
                d = (double)w[c * n + k] - (double)weff;
            }
            ds[a][kk] = d;
        }
        __syncthreads();
        const int kend = n - k0 < 64 ? n - k0 : 64;
        for (int kk = 0; kk < kend; ++kk) acc = acc + xs[tr][kk] * ds[tc][kk];
        __syncthreads();
    }
    const int64_t r = r0 + tr, c = c0 + tc;
    if (r < t && c < n_out) y[c * t + r] = acc;
}

// part[c] = sum_r y[c][r]^2 in token order.
__global__ __launch_bounds__(kThreads) void awq_channel_loss_kernel(const double *__restrict__ y, int64_t t,
                                                                    int64_t n_out, double *__restrict__ part)
{
    const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (c >= n_out) return;
    double acc = 0.0;
    for (int64_t r = 0; r < t; ++r) {
        const double v = y[c * t + r];
        acc += v * v;
    }
    part[c] = acc;
}

// loss[index] = sum_c part[c] in channel order.
__global__ void awq_total_kernel(const double *__restrict__ part, int64_t n_out, int index, double *__restrict__ loss)
{
    double acc = 0.0;
    for (int64_t c = 0; c < n_out; ++c) acc += part[c];
    loss[index] = acc;
}

// The first smallest loss; losses also exported as fp32 when asked for.
__global__ void awq_argmin_kernel(const double *__restrict__ loss, int count, int32_t *__restrict__ best,
                                  float *__restrict__ loss_out)
{
    int b = 0;
    for (int i = 1; i < count; ++i)
        if (loss[i] < loss[b]) b = i;
    *best = b;
    if (loss_out)
        for (int i = 0; i < count; ++i) loss_out[i] = (float)loss[i];
}

unsigned blocks_for(int64_t work) { return (unsigned)((work + kThreads - 1) / kThreads); }

}  // namespace

// Workspace layout (bytes, each piece 256-byte aligned).
static int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

int64_t gptq_factor_workspace(int64_t n) { return 2 * align256(n * n * 8); }

int64_t gptq_loop_workspace(int64_t n_out, int64_t n)
{
    return align256(n_out * n * 4) + align256(n_out * kBlock * 4) + align256(n_out * 8);
}

hipError_t gptq_launch_factor(const uint16_t *x, int64_t t, int n, double damp, void *workspace, float *u,
                              hipStream_t stream)
{
    double *S = static_cast<double *>(workspace);
    double *M = reinterpret_cast<double *>(static_cast<char *>(workspace) + align256((int64_t)n * n * 8));
    const int tiles = (n + 31) / 32;
    hessian_kernel<<<(unsigned)((int64_t)tiles * (tiles + 1) / 2), kThreads, 0, stream>>>(x, t, n, S);
    damp_kernel<<<1, kThreads, 0, stream>>>(S, n, damp);
    for (int j = 0; j < n; ++j) {
        const int rest = n - j - 1;
        if (rest > 0) chol_scale_kernel<<<blocks_for(rest), kThreads, 0, stream>>>(S, n, j);
        chol_update_kernel<<<dim3(blocks_for(rest > 0 ? rest : 1), (unsigned)(rest > 0 ? rest : 1)), kThreads, 0,
                             stream>>>(S, n, j);
    }
    identity_kernel<<<blocks_for((int64_t)n * n), kThreads, 0, stream>>>(M, n);
    for (int j = 0; j < n; ++j) {
        inv_scale_kernel<<<blocks_for(j + 1), kThreads, 0, stream>>>(S, M, n, j);
        if (j + 1 < n)
            inv_update_kernel<<<dim3(blocks_for(j + 1), (unsigned)(n - j - 1)), kThreads, 0, stream>>>(S, M, n, j);
    }
    u_from_inverse_kernel<<<blocks_for((int64_t)n * n), kThreads, 0, stream>>>(M, n, u);
    return hipGetLastError();
}

template <int BITS, bool SYM>
static hipError_t gptq_blocks(float *W, const float *u, int64_t n_out, int n, int group_size, float *E,
                              float *SZ, uint32_t *qweight, uint16_t *scales, uint16_t *zeros, hipStream_t stream)
{
    constexpr size_t kBlockLds = (size_t)(kBlock * 64 + kBlock * (kBlock + 1)) * sizeof(float);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void *>(gptq_block_kernel<BITS, SYM>), hipFuncAttributeMaxDynamicSharedMemorySize,
        (int)kBlockLds);
    if (attr != hipSuccess) return attr;
    for (int b0 = 0; b0 < n; b0 += kBlock) {
        const int b1 = b0 + kBlock < n ? b0 + kBlock : n;
        gptq_block_kernel<BITS, SYM><<<(unsigned)((n_out + 63) / 64), 64, kBlockLds, stream>>>(
            W, u, n_out, n, b0, b1, group_size, E, SZ, qweight, scales, zeros);
        if (b1 < n)
            gptq_trailing_kernel<<<dim3((unsigned)((n_out + 63) / 64), (unsigned)((n - b1 + 31) / 32)), kThreads, 0,
                                   stream>>>(W, u, E, n_out, n, b0, b1);
    }
    return hipSuccess;
}

hipError_t gptq_launch_loop(const float *w, const float *u, int64_t n_out, int n, int group_size, int bits,
                            bool symmetric, void *workspace, uint32_t *qweight, uint16_t *scales, uint16_t *zeros,
                            hipStream_t stream)
{
    float *W = static_cast<float *>(workspace);
    float *E = reinterpret_cast<float *>(static_cast<char *>(workspace) + align256(n_out * n * 4));
    float *SZ = reinterpret_cast<float *>(reinterpret_cast<char *>(E) + align256(n_out * kBlock * 4));
    hipError_t e = hipMemcpyAsync(W, w, (size_t)(n_out * n) * 4, hipMemcpyDeviceToDevice, stream);
    if (e != hipSuccess) return e;
    if (bits == 8)
        e = symmetric ? gptq_blocks<8, true>(W, u, n_out, n, group_size, E, SZ, qweight, scales, zeros, stream)
                      : gptq_blocks<8, false>(W, u, n_out, n, group_size, E, SZ, qweight, scales, zeros, stream);
    else
        e = symmetric ? gptq_blocks<4, true>(W, u, n_out, n, group_size, E, SZ, qweight, scales, zeros, stream)
                      : gptq_blocks<4, false>(W, u, n_out, n, group_size, E, SZ, qweight, scales, zeros, stream);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

int64_t awq_workspace(int64_t n_out, int64_t n, int64_t t, int n_grid, int group_size)
{
    return align256(n * 8) + align256(n * 4) + 2 * align256(n_out * n * 4) + align256(n_out * n) +
           2 * align256(n_out * (n / group_size) * 2) + align256(n_out * t * 8) + align256(n_out * 8) +
           align256((int64_t)(n_grid + 1) * 8) + align256(4);
}

hipError_t awq_launch(const float *w, const uint16_t *x, int64_t t, int64_t n_out, int n, int group_size, int bits,
                      bool symmetric, int n_grid, void *workspace, uint32_t *qweight, uint16_t *scales,
                      uint16_t *zeros, float *s_out, int32_t *best_out, float *losses_out, hipStream_t stream)
{
    char *p = static_cast<char *>(workspace);
    auto take = [&](int64_t bytes) { char *r = p; p += align256(bytes); return r; };
    double *mean = reinterpret_cast<double *>(take((int64_t)n * 8));
    float *s = reinterpret_cast<float *>(take((int64_t)n * 4));
    float *ws = reinterpret_cast<float *>(take(n_out * n * 4));
    float *deq = reinterpret_cast<float *>(take(n_out * n * 4));
    uint32_t *qtmp = reinterpret_cast<uint32_t *>(take(n_out * n));
    uint16_t *stmp = reinterpret_cast<uint16_t *>(take(n_out * (n / group_size) * 2));
    uint16_t *ztmp = reinterpret_cast<uint16_t *>(take(n_out * (n / group_size) * 2));
    double *y = reinterpret_cast<double *>(take(n_out * t * 8));
    double *part = reinterpret_cast<double *>(take(n_out * 8));
    double *loss = reinterpret_cast<double *>(take((int64_t)(n_grid + 1) * 8));
    int32_t *best = reinterpret_cast<int32_t *>(take(4));
    const int64_t total = n_out * n;
    act_mean_kernel<<<blocks_for(n), kThreads, 0, stream>>>(x, t, n, mean);
    for (int i = 0; i <= n_grid; ++i) {
        awq_scales_kernel<<<blocks_for(n), kThreads, 0, stream>>>(mean, n, i, n_grid, nullptr, s);
        scale_columns_kernel<<<blocks_for(total), kThreads, 0, stream>>>(w, s, total, n, ws);
        hipError_t e = q4_launch_quantize_pack(ws, n_out, n, group_size, bits, symmetric, qtmp, stmp, ztmp, stream);
        if (e != hipSuccess) return e;
        e = q4_launch_dequant(qtmp, stmp, ztmp, n_out, n, group_size, bits, deq, stream);
        if (e != hipSuccess) return e;
        awq_out_err_kernel<<<dim3((unsigned)((t + 15) / 16), (unsigned)((n_out + 15) / 16)), kThreads, 0, stream>>>(
            x, w, deq, s, t, n_out, n, y);
        awq_channel_loss_kernel<<<blocks_for(n_out), kThreads, 0, stream>>>(y, t, n_out, part);
        awq_total_kernel<<<1, 1, 0, stream>>>(part, n_out, i, loss);
    }
    awq_argmin_kernel<<<1, 1, 0, stream>>>(loss, n_grid + 1, best, losses_out);
    awq_scales_kernel<<<blocks_for(n), kThreads, 0, stream>>>(mean, n, 0, n_grid, best, s_out);
    scale_columns_kernel<<<blocks_for(total), kThreads, 0, stream>>>(w, s_out, total, n, ws);
    hipError_t e = q4_launch_quantize_pack(ws, n_out, n, group_size, bits, symmetric, qweight, scales, zeros, stream);
    if (e != hipSuccess) return e;
    if (best_out) {
        e = hipMemcpyAsync(best_out, best, 4, hipMemcpyDeviceToDevice, stream);
        if (e != hipSuccess) return e;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scratch of the no-allocation GPTQ column loop: a file-scope device array,
// one copy per GPU, held until the process ends.  Host code never uses the
// array's name as an address: each device's copy is looked up once with
// hipGetSymbolAddress and that pointer is what the launches receive.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[kGptqNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];
}  // namespace

hipError_t gptq_noalloc_scratch(hipStream_t stream, void **ptr)
{
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}
