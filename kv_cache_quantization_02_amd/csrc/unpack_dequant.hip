// unpack_dequant.hip - dense bf16 view of a VAR-Q packed cache (gfx950).
//
// README "Memory-Efficient Runtime" (the unpack+dequant operator) and project
// page Fig. 8: field i of word w is the b-bit two's complement code of channel
// w*cpw + i; the value is bf16_rne(fp32(q) * s[block(t), channel]).
//
// One thread writes one 16-byte chunk (8 channels) of one output row, so the
// stores of a wave are contiguous; the 1-3 words a chunk needs are read from
// their planes. ROPE (pre-RoPE quantization, project page Appendix F): the
// chunk's four channel pairs (2i, 2i+1) are then rotated by cos/sin[t, i]
// (fp32, each product and the sum rounded) and rounded to bf16 again.
#include "varq_device.h"

namespace varq {

constexpr int UD_THREADS = 256;

template <int BITS, bool ROPE>
__global__ __launch_bounds__(UD_THREADS) void unpack_dequant_kernel(const UnpackArgs a) {
    constexpr int CPW = 32 / BITS;
    constexpr uint32_t MASK = (1u << BITS) - 1u;
    constexpr int SHIFT = 32 - BITS;

    __shared__ int32_t off[VARQ_MAX_GROUPS_DEV + 1];
    for (int i = threadIdx.x; i <= a.G; i += UD_THREADS) off[i] = a.off[i];
    __syncthreads();

    const int chunks = a.D >> 3;
    const int64_t item = (int64_t)blockIdx.x * UD_THREADS + threadIdx.x;
    const int64_t total = (int64_t)a.B * a.H * a.L * chunks;
    if (item >= total) return;
    const int j = (int)(item % chunks);
    const int64_t rowid = item / chunks;             // (b*H + h)*L + t
    const int64_t t = rowid % a.L;
    const int64_t bh = rowid / a.L;

    // block of token t (binary search)
    int lo = 0, hi = a.G;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (off[mid] <= t) lo = mid; else hi = mid;
    }
    const float *srow = a.scales + (bh * a.G_cap + lo) * a.D;
    const uint32_t *planes = a.packed + bh * a.W * a.L_cap + t;

    uint32_t outw[4];
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
        uint32_t bits2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int c = 8 * j + k + e;
            const int w = c / CPW, i = c % CPW;
            const uint32_t word = planes[(int64_t)w * a.L_cap];
            const int32_t q = (int32_t)(word << (SHIFT - i * BITS)) >> SHIFT;   // sign-extend field i
            (void)MASK;
            bits2[e] = dequant_bits(q, srow[c]);
        }
        if constexpr (ROPE) {
            const int64_t trow = t * (a.D >> 1) + 4 * j + (k >> 1);
            const float c = a.rcos[trow], s = a.rsin[trow];
            const float x0 = u2f(bits2[0] << 16), x1 = u2f(bits2[1] << 16);
            const float c0 = x0 * c, c1 = x1 * s, c2 = x0 * s, c3 = x1 * c;
            bits2[0] = bf16_bits_rne(c0 - c1);
            bits2[1] = bf16_bits_rne(c2 + c3);
        }
        outw[k >> 1] = bits2[0] | (bits2[1] << 16);
    }
    uint4 *dst = reinterpret_cast<uint4 *>(a.out + rowid * a.D + 8 * j);
    *dst = make_uint4(outw[0], outw[1], outw[2], outw[3]);
}

template <int BITS>
static hipError_t launch_ud(const UnpackArgs &a, hipStream_t st) {
    const int64_t total = (int64_t)a.B * a.H * a.L * (a.D >> 3);
    const int64_t grid = (total + UD_THREADS - 1) / UD_THREADS;
    if (a.rcos)
        hipLaunchKernelGGL((unpack_dequant_kernel<BITS, true>), dim3((unsigned)grid), dim3(UD_THREADS), 0, st, a);
    else
        hipLaunchKernelGGL((unpack_dequant_kernel<BITS, false>), dim3((unsigned)grid), dim3(UD_THREADS), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_unpack_dequant(const UnpackArgs &a, int bits, hipStream_t st) {
    switch (bits) {
        case 2: return launch_ud<2>(a, st);
        case 3: return launch_ud<3>(a, st);
        case 4: return launch_ud<4>(a, st);
        case 5: return launch_ud<5>(a, st);
        case 6: return launch_ud<6>(a, st);
        case 7: return launch_ud<7>(a, st);
        case 8: return launch_ud<8>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace varq
