// q4_quantize.hip -- group-wise INT4 quantization + packing, and dequantization.
//
// Quantizer: [Guide] §2.1 (uniform affine map q = clamp(round(x/s) + z) with
// min-max calibration, s floored at 1e-8), [Path] §2.1 (z and the codes are
// clipped to the code range), [Guide] §2.2 (one scale/zero-point per group of
// input elements of an output channel, fp16 storage).
// Dequantizer: [Guide] §2.1 (x_hat = s (q - z), float32 result), [Zero] §2.
//
// This translation unit is built with -ffp-contract=off and correctly rounded
// fp32 division so that every step is one IEEE binary32 operation with
// round-to-nearest-even: the packed codes, scales and zero-points are then
// identical bit for bit to any other IEEE evaluation of the same steps.
//
// Work layout.  Groups never straddle rows (n_in % group_size == 0), so the
// weight matrix is treated as one flat array of n_out*n_in/8 packed words.
// Each lane owns one word: it reads its eight fp32 weights with two 16-byte
// loads (consecutive lanes read consecutive 32-byte spans), the group_size/8
// lanes of a group combine their range with a butterfly of lane shuffles,
// each lane computes the group's s and z redundantly, codes and packs its own
// eight weights and stores one 32-bit word (one 256-byte run per wave).  The
// first lane of each group stores the fp16 scale and zero-point.
#include "q4_device.h"
#include "q4_launch.h"

namespace {

template <int LANES, bool SYMMETRIC>
__global__ __launch_bounds__(256) void quantize_pack_kernel(
    const float *__restrict__ w, uint32_t *__restrict__ qweight,
    uint16_t *__restrict__ scales, uint16_t *__restrict__ zeros, int64_t n_words)
{
    const int64_t word = (int64_t)blockIdx.x * 256 + threadIdx.x;
    // Whole groups are either inside or outside the array, and every group
    // starts at a multiple of LANES, so lanes past the end only ever combine
    // with each other.  They read the last word and store nothing.
    const bool active = word < n_words;
    const int64_t src_word = active ? word : n_words - 1;

    const float4 *src = reinterpret_cast<const float4 *>(w + src_word * 8);
    const float4 lo = src[0], hi = src[1];
    const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};

    float s, zf;
    uint32_t packed = 0;
    if (SYMMETRIC) {
        float amax = fabsf(v[0]);
#pragma unroll
        for (int i = 1; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
        for (int off = 1; off < LANES; off <<= 1)
            amax = fmaxf(amax, __shfl_xor(amax, off));
        s = amax / 7.0f;
        if (s < 1e-8f) s = 1e-8f;
        zf = 8.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float q = fminf(fmaxf(rintf(v[i] / s), -8.0f), 7.0f);
            packed |= (uint32_t)((int)q + 8) << (4 * i);
        }
    } else {
        float mn = v[0], mx = v[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) {
            mn = fminf(mn, v[i]);
            mx = fmaxf(mx, v[i]);
        }
#pragma unroll
        for (int off = 1; off < LANES; off <<= 1) {
            mn = fminf(mn, __shfl_xor(mn, off));
            mx = fmaxf(mx, __shfl_xor(mx, off));
        }
        // The sign of a zero min or max cannot change s, z or any code.
        s = (mx - mn) / 15.0f;
        if (s < 1e-8f) s = 1e-8f;
        zf = fminf(fmaxf(rintf(-mn / s), 0.0f), 15.0f);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float q = fminf(fmaxf(rintf(v[i] / s) + zf, 0.0f), 15.0f);
            packed |= (uint32_t)q << (4 * i);
        }
    }

    if (active) {
        qweight[word] = packed;
        if ((word & (LANES - 1)) == 0) {
            const int64_t group = word / LANES;
            scales[group] = bitcast<uint16_t>((_Float16)s);
            zeros[group] = bitcast<uint16_t>((_Float16)zf);
        }
    }
}

// One lane per packed word: eight fp32 outputs written as two 16-byte stores.
__global__ __launch_bounds__(256) void dequant_kernel(
    const uint32_t *__restrict__ qweight, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ zeros, float *__restrict__ out, int64_t n_words,
    int group_shift_words)
{
    const int64_t word = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (word >= n_words) return;
    const uint32_t q = qweight[word];
    const int64_t group = word >> group_shift_words;
    const float s = half_bits_to_float(scales[group]);
    const int z = (int)half_bits_to_float(zeros[group]);
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = s * (float)((int)((q >> (4 * i)) & 0xFu) - z);
    float4 *dst = reinterpret_cast<float4 *>(out + word * 8);
    dst[0] = make_float4(r[0], r[1], r[2], r[3]);
    dst[1] = make_float4(r[4], r[5], r[6], r[7]);
}

template <bool SYMMETRIC>
hipError_t launch_quantize(const float *w, int64_t n_words, int group_size,
                           uint32_t *qweight, uint16_t *scales, uint16_t *zeros,
                           hipStream_t stream)
{
    const dim3 grid((unsigned)((n_words + 255) / 256)), block(256);
    switch (group_size) {
    case 32:
        quantize_pack_kernel<4, SYMMETRIC><<<grid, block, 0, stream>>>(w, qweight, scales, zeros, n_words);
        break;
    case 64:
        quantize_pack_kernel<8, SYMMETRIC><<<grid, block, 0, stream>>>(w, qweight, scales, zeros, n_words);
        break;
    case 128:
        quantize_pack_kernel<16, SYMMETRIC><<<grid, block, 0, stream>>>(w, qweight, scales, zeros, n_words);
        break;
    case 256:
        quantize_pack_kernel<32, SYMMETRIC><<<grid, block, 0, stream>>>(w, qweight, scales, zeros, n_words);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t q4_launch_quantize_pack(const float *w, int64_t n_out, int64_t n_in,
                                   int group_size, bool symmetric, uint32_t *qweight,
                                   uint16_t *scales, uint16_t *zeros, hipStream_t stream)
{
    const int64_t n_words = n_out * (n_in / 8);
    return symmetric
               ? launch_quantize<true>(w, n_words, group_size, qweight, scales, zeros, stream)
               : launch_quantize<false>(w, n_words, group_size, qweight, scales, zeros, stream);
}

hipError_t q4_launch_dequant(const uint32_t *qweight, const uint16_t *scales,
                             const uint16_t *zeros, int64_t n_out, int64_t n_in,
                             int group_size, float *out, hipStream_t stream)
{
    const int64_t n_words = n_out * (n_in / 8);
    int shift = 0;
    while ((8 << shift) < group_size) ++shift;       // words per group = 2^shift
    const dim3 grid((unsigned)((n_words + 255) / 256)), block(256);
    dequant_kernel<<<grid, block, 0, stream>>>(qweight, scales, zeros, out, n_words, shift);
    return hipGetLastError();
}
