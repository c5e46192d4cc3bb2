// q4_quantize.hip -- group-wise (or per-channel) INT4 / INT8 quantization +
// packing, and dequantization.
//
// Quantizer: [Guide] §2.1 (uniform affine map q = clamp(round(x/s) + z) with
// min-max calibration, s floored at 1e-8; b-bit ranges: asymmetric
// s = (max - min)/(2^b - 1), symmetric s = max|x|/(2^(b-1) - 1)), [Path] §2.1
// (z and the codes are clipped to the code range), [Guide] §2.2 (one
// scale/zero-point per group of input elements of an output channel, or per
// output channel -- the usual choice for INT8 weights -- fp16 storage),
// [Guide] §2.3 (W4A16 and W8A16).
// Dequantizer: [Guide] §2.1 (x_hat = s (q - z), float32 result), [Zero] §2.
//
// This translation unit is built with -ffp-contract=off and correctly rounded
// fp32 division so that every step is one IEEE binary32 operation with
// round-to-nearest-even: the packed codes, scales and zero-points are then
// identical bit for bit to any other IEEE evaluation of the same steps.
//
// Packing: a 32-bit word holds 32/BITS codes, element t of the word in bits
// BITS*t.. (8 nibbles or 4 bytes); symmetric codes q are stored as
// q + 2^(BITS-1) with a stored zero-point of 2^(BITS-1).
//
// Work layout, groups of 32..256 elements.  Groups never straddle rows
// (n_in % group_size == 0), so the weight matrix is treated as one flat array
// of packed words.  Each lane owns one word: it reads its 32/BITS fp32
// weights with 16-byte loads (consecutive lanes read consecutive spans), the
// lanes of a group combine their range with a butterfly of lane shuffles,
// each lane computes the group's s and z redundantly, codes and packs its own
// weights and stores one 32-bit word.  The first lane of each group stores
// the fp16 scale and zero-point.
// Per-channel (the group is a whole row of any length): one workgroup per
// row reduces the row's range across its waves through LDS, then codes and
// packs the row in a second pass over it (the row is then cache-resident).
#include "q4_device.h"
#include "q4_launch.h"

namespace {

template <int BITS>
struct Codes {
    static constexpr int PER_WORD = 32 / BITS;
    static constexpr float ASYM_MAX = (float)((1 << BITS) - 1);        // 15 or 255
    static constexpr float SYM_MAX = (float)((1 << (BITS - 1)) - 1);   // 7 or 127
    static constexpr float SYM_MIN = -(float)(1 << (BITS - 1));        // -8 or -128
    static constexpr int OFFSET = 1 << (BITS - 1);                     // 8 or 128
};

// Scale and zero-point of a group from its reduced range.
template <int BITS, bool SYMMETRIC>
__device__ __forceinline__ void scale_zero(float a, float b, float &s, float &zf)
{
    using C = Codes<BITS>;
    if (SYMMETRIC) {                        // a = max|w|
        s = a / C::SYM_MAX;
        if (s < 1e-8f) s = 1e-8f;
        zf = (float)C::OFFSET;
    } else {                                // a = min, b = max; a zero's sign cannot matter
        s = (b - a) / C::ASYM_MAX;
        if (s < 1e-8f) s = 1e-8f;
        zf = fminf(fmaxf(rintf(-a / s), 0.0f), C::ASYM_MAX);
    }
}

// Codes of one word's weights, packed.
template <int BITS, bool SYMMETRIC>
__device__ __forceinline__ uint32_t pack_word(const float *v, float s, float zf)
{
    using C = Codes<BITS>;
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < C::PER_WORD; ++i) {
        if (SYMMETRIC) {
            const float q = fminf(fmaxf(rintf(v[i] / s), C::SYM_MIN), C::SYM_MAX);
            packed |= (uint32_t)((int)q + C::OFFSET) << (BITS * i);
        } else {
            const float q = fminf(fmaxf(rintf(v[i] / s) + zf, 0.0f), C::ASYM_MAX);
            packed |= (uint32_t)q << (BITS * i);
        }
    }
    return packed;
}

template <int BITS>
__device__ __forceinline__ void load_word(const float *w, int64_t word, float *v)
{
    const float4 *src = reinterpret_cast<const float4 *>(w + word * Codes<BITS>::PER_WORD);
#pragma unroll
    for (int j = 0; j < Codes<BITS>::PER_WORD / 4; ++j) {
        const float4 f = src[j];
        v[4 * j] = f.x;
        v[4 * j + 1] = f.y;
        v[4 * j + 2] = f.z;
        v[4 * j + 3] = f.w;
    }
}

template <int LANES, bool SYMMETRIC, int BITS>
__global__ __launch_bounds__(256) void quantize_pack_kernel(
    const float *__restrict__ w, uint32_t *__restrict__ qweight,
    uint16_t *__restrict__ scales, uint16_t *__restrict__ zeros, int64_t n_words)
{
    constexpr int PER_WORD = Codes<BITS>::PER_WORD;
    const int64_t word = (int64_t)blockIdx.x * 256 + threadIdx.x;
    // Whole groups are either inside or outside the array, and every group
    // starts at a multiple of LANES, so lanes past the end only ever combine
    // with each other.  They read the last word and store nothing.
    const bool active = word < n_words;
    float v[PER_WORD];
    load_word<BITS>(w, active ? word : n_words - 1, v);

    float a, b;
    if (SYMMETRIC) {
        a = fabsf(v[0]);
#pragma unroll
        for (int i = 1; i < PER_WORD; ++i) a = fmaxf(a, fabsf(v[i]));
#pragma unroll
        for (int off = 1; off < LANES; off <<= 1) a = fmaxf(a, __shfl_xor(a, off));
        b = a;
    } else {
        a = v[0];
        b = v[0];
#pragma unroll
        for (int i = 1; i < PER_WORD; ++i) {
            a = fminf(a, v[i]);
            b = fmaxf(b, v[i]);
        }
#pragma unroll
        for (int off = 1; off < LANES; off <<= 1) {
            a = fminf(a, __shfl_xor(a, off));
            b = fmaxf(b, __shfl_xor(b, off));
        }
    }
    float s, zf;
    scale_zero<BITS, SYMMETRIC>(a, b, s, zf);
    const uint32_t packed = pack_word<BITS, SYMMETRIC>(v, s, zf);

    if (active) {
        qweight[word] = packed;
        if ((word & (LANES - 1)) == 0) {
            const int64_t group = word / LANES;
            scales[group] = bitcast<uint16_t>((_Float16)s);
            zeros[group] = bitcast<uint16_t>((_Float16)zf);
        }
    }
}

// Per-channel: one workgroup of 256 lanes per row of `words` packed words.
template <bool SYMMETRIC, int BITS>
__global__ __launch_bounds__(256) void quantize_rows_kernel(
    const float *__restrict__ w, uint32_t *__restrict__ qweight,
    uint16_t *__restrict__ scales, uint16_t *__restrict__ zeros, int64_t words)
{
    constexpr int PER_WORD = Codes<BITS>::PER_WORD;
    __shared__ float red_a[4], red_b[4];
    const int64_t row = blockIdx.x;
    const float *wr = w + row * words * PER_WORD;
    uint32_t *qr = qweight + row * words;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    float a = SYMMETRIC ? 0.0f : INFINITY, b = SYMMETRIC ? 0.0f : -INFINITY;
    for (int64_t i = tid; i < words; i += 256) {
        float v[PER_WORD];
        load_word<BITS>(wr, i, v);
#pragma unroll
        for (int j = 0; j < PER_WORD; ++j) {
            if (SYMMETRIC) {
                a = fmaxf(a, fabsf(v[j]));
            } else {
                a = fminf(a, v[j]);
                b = fmaxf(b, v[j]);
            }
        }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        a = SYMMETRIC ? fmaxf(a, __shfl_xor(a, off)) : fminf(a, __shfl_xor(a, off));
        b = fmaxf(b, __shfl_xor(b, off));
    }
    if (lane == 0) {
        red_a[wave] = a;
        red_b[wave] = b;
    }
    __syncthreads();
    a = red_a[0];
    b = red_b[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) {
        a = SYMMETRIC ? fmaxf(a, red_a[i]) : fminf(a, red_a[i]);
        b = fmaxf(b, red_b[i]);
    }
    float s, zf;
    scale_zero<BITS, SYMMETRIC>(a, b, s, zf);
    for (int64_t i = tid; i < words; i += 256) {
        float v[PER_WORD];
        load_word<BITS>(wr, i, v);
        qr[i] = pack_word<BITS, SYMMETRIC>(v, s, zf);
    }
    if (tid == 0) {
        scales[row] = bitcast<uint16_t>((_Float16)s);
        zeros[row] = bitcast<uint16_t>((_Float16)zf);
    }
}

// One lane per packed word: its fp32 outputs written as 16-byte stores.  The
// group of a word is word >> shift, or its row (word / words_per_row) for
// per-channel weights.
template <int BITS, bool PER_CHANNEL>
__global__ __launch_bounds__(256) void dequant_kernel(
    const uint32_t *__restrict__ qweight, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ zeros, float *__restrict__ out, int64_t n_words,
    int group_shift_words, int64_t words_per_row)
{
    constexpr int PER_WORD = Codes<BITS>::PER_WORD;
    constexpr uint32_t MASK = (1u << BITS) - 1u;
    const int64_t word = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (word >= n_words) return;
    const uint32_t q = qweight[word];
    const int64_t group = PER_CHANNEL ? word / words_per_row : word >> group_shift_words;
    const float s = half_bits_to_float(scales[group]);
    const int z = (int)half_bits_to_float(zeros[group]);
    float r[PER_WORD];
#pragma unroll
    for (int i = 0; i < PER_WORD; ++i) r[i] = s * (float)((int)((q >> (BITS * i)) & MASK) - z);
    float4 *dst = reinterpret_cast<float4 *>(out + word * PER_WORD);
#pragma unroll
    for (int j = 0; j < PER_WORD / 4; ++j)
        dst[j] = make_float4(r[4 * j], r[4 * j + 1], r[4 * j + 2], r[4 * j + 3]);
}

// INT4 dequantization: one lane per 16-bit half word (four codes) and one
// float4 of output, ITEMS runs of 256 lanes per workgroup, so every store
// instruction of a wave writes 1 KiB of contiguous output (one lane per
// packed word would split each 32-byte output span over two half-covered
// store instructions, which HBM serves markedly slower).
// The group of half word f is f >> shift, or its row (f / per_row) for
// per-channel weights.
template <int ITEMS, bool PER_CHANNEL>
__global__ __launch_bounds__(256) void dequant4_kernel(
    const uint16_t *__restrict__ q16, const uint16_t *__restrict__ scales,
    const uint16_t *__restrict__ zeros, float *__restrict__ out, int64_t n4, int group_shift4, int64_t per_row)
{
    const int64_t base = (int64_t)blockIdx.x * (256 * ITEMS) + threadIdx.x;
    uint32_t q[ITEMS];
    int64_t grp[ITEMS];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int64_t f = base + (int64_t)it * 256;
        const int64_t fc = f < n4 ? f : n4 - 1;
        q[it] = q16[fc];
        grp[it] = PER_CHANNEL ? fc / per_row : fc >> group_shift4;
    }
    float4 *dst = reinterpret_cast<float4 *>(out);
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int64_t f = base + (int64_t)it * 256;
        const float sc = half_bits_to_float(scales[grp[it]]);
        const int z = (int)half_bits_to_float(zeros[grp[it]]);
        float r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = sc * (float)((int)((q[it] >> (4 * i)) & 15u) - z);
        if (f < n4) dst[f] = make_float4(r[0], r[1], r[2], r[3]);
    }
}

template <bool SYMMETRIC, int BITS>
hipError_t launch_quantize(const float *w, int64_t n_out, int64_t n_in, int group_size,
                           uint32_t *qweight, uint16_t *scales, uint16_t *zeros,
                           hipStream_t stream)
{
    constexpr int PER_WORD = Codes<BITS>::PER_WORD;
    const int64_t n_words = n_out * (n_in / PER_WORD);
    const bool pow2_group = group_size >= 32 && group_size <= 256 && (group_size & (group_size - 1)) == 0;
    if (!pow2_group) {                                   // per-channel rows of any other length
        quantize_rows_kernel<SYMMETRIC, BITS><<<dim3((unsigned)n_out), dim3(256), 0, stream>>>(
            w, qweight, scales, zeros, n_in / PER_WORD);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((n_words + 255) / 256)), block(256);
    // lanes per group = group_size / PER_WORD
    switch (group_size / PER_WORD) {
#define Q4_Q(L)                                                                                       \
    case L:                                                                                           \
        quantize_pack_kernel<L, SYMMETRIC, BITS><<<grid, block, 0, stream>>>(w, qweight, scales, zeros, \
                                                                             n_words);                \
        break;
        Q4_Q(4)
        Q4_Q(8)
        Q4_Q(16)
        Q4_Q(32)
        Q4_Q(64)
#undef Q4_Q
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_dequant(const uint32_t *qweight, const uint16_t *scales, const uint16_t *zeros,
                          int64_t n_out, int64_t n_in, int group_size, float *out, hipStream_t stream)
{
    constexpr int PER_WORD = Codes<BITS>::PER_WORD;
    const int64_t words_per_row = n_in / PER_WORD;
    const int64_t n_words = n_out * words_per_row;
    if constexpr (BITS == 4) {
        constexpr int ITEMS = 4;
        const int64_t n4 = n_words * 2;
        const dim3 grid4((unsigned)((n4 + 256 * ITEMS - 1) / (256 * ITEMS))), block4(256);
        const uint16_t *q16 = reinterpret_cast<const uint16_t *>(qweight);
        const int per_group = group_size / 4;
        if ((per_group & (per_group - 1)) == 0) {
            int shift = 0;
            while ((1 << shift) < per_group) ++shift;
            dequant4_kernel<ITEMS, false><<<grid4, block4, 0, stream>>>(q16, scales, zeros, out, n4, shift, n_in / 4);
        } else {                                        // per-channel with a row of other length
            dequant4_kernel<ITEMS, true><<<grid4, block4, 0, stream>>>(q16, scales, zeros, out, n4, 0, n_in / 4);
        }
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((n_words + 255) / 256)), block(256);
    const int words_per_group = group_size / PER_WORD;
    if ((words_per_group & (words_per_group - 1)) == 0) {
        int shift = 0;
        while ((1 << shift) < words_per_group) ++shift;
        dequant_kernel<BITS, false><<<grid, block, 0, stream>>>(qweight, scales, zeros, out, n_words, shift,
                                                                words_per_row);
    } else {                                            // per-channel with a row of other length
        dequant_kernel<BITS, true><<<grid, block, 0, stream>>>(qweight, scales, zeros, out, n_words, 0,
                                                               words_per_row);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t q4_launch_quantize_pack(const float *w, int64_t n_out, int64_t n_in, int group_size,
                                   int bits, bool symmetric, uint32_t *qweight, uint16_t *scales,
                                   uint16_t *zeros, hipStream_t stream)
{
    if (bits == 8)
        return symmetric ? launch_quantize<true, 8>(w, n_out, n_in, group_size, qweight, scales, zeros, stream)
                         : launch_quantize<false, 8>(w, n_out, n_in, group_size, qweight, scales, zeros, stream);
    return symmetric ? launch_quantize<true, 4>(w, n_out, n_in, group_size, qweight, scales, zeros, stream)
                     : launch_quantize<false, 4>(w, n_out, n_in, group_size, qweight, scales, zeros, stream);
}

hipError_t q4_launch_dequant(const uint32_t *qweight, const uint16_t *scales,
                             const uint16_t *zeros, int64_t n_out, int64_t n_in,
                             int group_size, int bits, float *out, hipStream_t stream)
{
    return bits == 8 ? launch_dequant<8>(qweight, scales, zeros, n_out, n_in, group_size, out, stream)
                     : launch_dequant<4>(qweight, scales, zeros, n_out, n_in, group_size, out, stream);
}
