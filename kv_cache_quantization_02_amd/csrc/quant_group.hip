// quant_group.hip - quantize+pack with the grouping variants of the VAR-Q
// project page's grouping ablation (Table 5) and error table (Table 1).
//
// The grouping decides which elements share one scale; the codes, their
// packing and the word layout [B, H, W, L_cap] are those of the channel x
// block cache. The "channel axis" is the hidden width H * D, so the groupings
// without it share a scale across heads. Compact fp32 scale layouts:
//   BLOCK       [B, G]      without channel axis (one scale per sequence and block)
//   TOKEN_HEAD  [B, H, L]   per-token & per-head
//   TOKEN       [B, L]      per-token
//   TENSOR      [1]         per-tensor
// (channel x block and "without block axis" are the main quant-pack kernel,
// the latter with one block [0, L).)
//
// Passes, all stream-ordered: (1) absmax of every token row (TOKEN_HEAD: of
// every (token, head) row) accumulated as fp32 bit patterns by atomic max
// (non-negative floats order like their bit patterns) after a segmented
// reduction within each wave over runs of equal row. TOKEN_HEAD and TOKEN
// accumulate straight into the scale buffer. BLOCK and TENSOR accumulate the
// token maxima in rows [0, L) of word plane 0 of head 0 of each sequence, which
// the last pass overwrites, and (1b) one work-group per block (BLOCK) or one
// for all (TENSOR) reduces them into the scale buffer; (2) every group's
// absmax becomes its scale s = fp32(absmax / qmax) in place; (3) one thread
// per (sequence, token, head, word) quantizes that word's channels with its
// group's scale and stores the word. This path exists to measure the
// groupings; it reads the input twice.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/varq.h"
#include "varq_device.h"
#include "varq_quant_math.h"

namespace varq {

namespace {

constexpr int GQ_THREADS = 256;

__device__ inline int block_of_token(const int32_t *off, int G, int64_t t) {
    int lo = 0, hi = G;                    // last g with off[g] <= t
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (off[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}

// Flat index into the compact scale layout of token t, head h of sequence b
// (the host checks that every count here fits 31 bits).
template <int MODE>
__device__ inline int group_id(const GroupArgs &a, const int32_t *off, int b, int t, int h) {
    if constexpr (MODE == VARQ_GROUP_BLOCK) return b * a.G + block_of_token(off, a.G, t);
    else if constexpr (MODE == VARQ_GROUP_TOKEN_HEAD) return (b * a.H + h) * a.L + t;
    else if constexpr (MODE == VARQ_GROUP_TOKEN) return b * a.L + t;
    else return 0;
}

// Clear `rows` runs of `len` words spaced `pitch` apart.
__global__ __launch_bounds__(GQ_THREADS) void group_clear_kernel(uint32_t *p, int64_t rows, int64_t len, int64_t pitch) {
    const int64_t n = rows * len;
    for (int64_t i = (int64_t)blockIdx.x * GQ_THREADS + threadIdx.x; i < n; i += (int64_t)gridDim.x * GQ_THREADS)
        p[(i / len) * pitch + i % len] = 0u;
}

// Pass 1: items of 8 channels in (b, t, h, chunk) order, one per thread and
// grid step; absmax bit patterns reduced over runs of equal row in a wave,
// then one atomic max per run into the row's accumulator.
template <int MODE>
__global__ __launch_bounds__(GQ_THREADS) void group_absmax_kernel(const GroupArgs a) {
    const int lpr = a.D >> 3;
    const int n_items = a.B * a.L * a.H * lpr;
    const int lane = threadIdx.x & 63;
    const int64_t plane_pitch = (int64_t)a.H * a.W * a.L_cap;     // words per sequence in `packed`
    // every wave runs the same number of iterations (the exchange below needs
    // all 64 lanes); items past the end carry an absmax of 0 and row -1
    const int stride = gridDim.x * GQ_THREADS;
    const int wave0 = blockIdx.x * GQ_THREADS + (threadIdx.x & ~63);
    for (int base = wave0; base < n_items; base += stride) {
        const int i = base + lane;
        uint32_t m = 0;
        int gid = -1;
        if (i < n_items) {
            const int chunk = i % lpr, r = i / lpr;
            const int h = r % a.H, bt = r / a.H;
            const int t = bt % a.L, b = bt / a.L;
            const uint4 w = *reinterpret_cast<const uint4 *>(a.x + b * a.sx_b + t * a.sx_l + h * a.sx_h + 8 * chunk);
            const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                m = max(m, (v[j] & 0x7FFFu) << 16);          // |low bf16| as fp32 bits
                m = max(m, v[j] & 0x7FFF0000u);             // |high bf16| as fp32 bits
            }
            gid = MODE == VARQ_GROUP_TOKEN_HEAD ? (b * a.H + h) * a.L + t : b * a.L + t;
        }
        // segmented maximum over runs of equal row (runs are contiguous in lanes)
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t mo = (uint32_t)__shfl_down((int)m, d);
            const int go = __shfl_down(gid, d);
            if (lane + d < 64 && go == gid) m = max(m, mo);
        }
        const int gprev = __shfl_up(gid, 1);
        if (gid >= 0 && (lane == 0 || gprev != gid)) {
            uint32_t *acc;
            if constexpr (MODE == VARQ_GROUP_TOKEN_HEAD || MODE == VARQ_GROUP_TOKEN) {
                acc = a.absmax + gid;
            } else {
                const int b = gid / a.L, t = gid - b * a.L;
                acc = a.packed + b * plane_pitch + t;
            }
            atomicMax(acc, m);
        }
    }
}

// Pass 1b (BLOCK, TENSOR): work-group x reduces the token maxima of block x
// (BLOCK, x = b * G + g) or of every token (TENSOR, one work-group).
template <int MODE>
__global__ __launch_bounds__(GQ_THREADS) void group_reduce_kernel(const GroupArgs a) {
    __shared__ uint32_t sh[GQ_THREADS / 64];
    const int64_t plane_pitch = (int64_t)a.H * a.W * a.L_cap;
    int b0 = 0, b1 = a.B, t0 = 0, t1 = a.L;
    if constexpr (MODE == VARQ_GROUP_BLOCK) {
        b0 = blockIdx.x / a.G;
        b1 = b0 + 1;
        const int g = blockIdx.x - b0 * a.G;
        t0 = a.off[g];
        t1 = a.off[g + 1];
    }
    uint32_t m = 0;
    for (int b = b0; b < b1; ++b)
        for (int t = t0 + threadIdx.x; t < t1; t += GQ_THREADS) m = max(m, a.packed[b * plane_pitch + t]);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d));
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < GQ_THREADS / 64; ++w) m = max(m, sh[w]);
        a.absmax[MODE == VARQ_GROUP_BLOCK ? blockIdx.x : 0] = m;
    }
}

// Pass 2: absmax bit pattern -> scale s = fp32(absmax / qmax), in place.
__global__ __launch_bounds__(GQ_THREADS) void group_scale_kernel(uint32_t *p, int64_t n, float qmax) {
    for (int64_t i = (int64_t)blockIdx.x * GQ_THREADS + threadIdx.x; i < n; i += (int64_t)gridDim.x * GQ_THREADS)
        p[i] = f2u(u2f(p[i]) / qmax);                         // IEEE fp32 division
}

// Pass 3: word w of (b, t, h), w fastest so that the threads of a row read it
// together. Fields LSB-first, two's complement, channels past D are zero.
template <int BITS, int MODE>
__global__ __launch_bounds__(GQ_THREADS) void group_quant_kernel(const GroupArgs a) {
    constexpr int CPW = 32 / BITS;
    constexpr uint32_t MASK = (1u << BITS) - 1u;
    __shared__ int32_t sh_off[257];
    for (int i = threadIdx.x; i <= a.G; i += GQ_THREADS) sh_off[i] = a.off[i];
    __syncthreads();
    const int n = a.B * a.L * a.H * a.W;
    const float *sc = reinterpret_cast<const float *>(a.absmax);
    for (int i = blockIdx.x * GQ_THREADS + threadIdx.x; i < n; i += gridDim.x * GQ_THREADS) {
        const int w = i % a.W, r = i / a.W;
        const int h = r % a.H, bt = r / a.H;
        const int t = bt % a.L, b = bt / a.L;
        const float s = sc[group_id<MODE>(a, sh_off, b, t, h)];
        const float y = recip_for_codes(s);
        const bool fast = fast_scale_ok(s);
        const uint16_t *row = a.x + b * a.sx_b + t * a.sx_l + h * a.sx_h;
        const int c0 = w * CPW;
        // the word's channels c0 .. c0 + CPW - 1 (those below D), widest loads
        // their alignment allows: c0 is a multiple of CPW and D of 8
        uint16_t xs[CPW];
        if constexpr (CPW % 8 == 0) {
#pragma unroll
            for (int j = 0; j < CPW / 8; ++j) {
                uint4 v = make_uint4(0, 0, 0, 0);
                if (c0 + 8 * j < a.D) v = *reinterpret_cast<const uint4 *>(row + c0 + 8 * j);
                const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) { xs[8 * j + 2 * k] = (uint16_t)u[k]; xs[8 * j + 2 * k + 1] = (uint16_t)(u[k] >> 16); }
            }
        } else if constexpr (CPW == 4) {
            const uint2 v = *reinterpret_cast<const uint2 *>(row + c0);
            xs[0] = (uint16_t)v.x; xs[1] = (uint16_t)(v.x >> 16); xs[2] = (uint16_t)v.y; xs[3] = (uint16_t)(v.y >> 16);
        } else if constexpr (CPW % 2 == 0) {
#pragma unroll
            for (int j = 0; j < CPW / 2; ++j) {
                uint32_t v = 0;
                if (c0 + 2 * j < a.D) v = *reinterpret_cast<const uint32_t *>(row + c0 + 2 * j);
                xs[2 * j] = (uint16_t)v; xs[2 * j + 1] = (uint16_t)(v >> 16);
            }
        } else {
#pragma unroll
            for (int k = 0; k < CPW; ++k) xs[k] = c0 + k < a.D ? row[c0 + k] : (uint16_t)0;
        }
        uint32_t word = 0;
#pragma unroll
        for (int k = 0; k < CPW; ++k) {
            uint32_t f = 0;
            if (c0 + k < a.D) {
                const float x = u2f((uint32_t)xs[k] << 16);
                f = (uint32_t)(fast ? code_fast(x, s, y) : code_exact(x, s)) & MASK;
            }
            word |= f << (k * BITS);
        }
        a.packed[((int64_t)(b * a.H + h) * a.W + w) * a.L_cap + t] = word;
    }
}

template <int MODE>
hipError_t run_group(const GroupArgs &a, int bits, int64_t n_scales, int grid_items, hipStream_t st) {
    const int64_t n_items = (int64_t)a.B * a.L * a.H * (a.D >> 3);
    const int64_t n_words = (int64_t)a.B * a.L * a.H * a.W;
    auto blocks = [](int64_t n, int cap) { return (int)std::max<int64_t>(1, std::min<int64_t>((n + GQ_THREADS - 1) / GQ_THREADS, cap)); };
    constexpr bool VIA_TOKENS = MODE == VARQ_GROUP_BLOCK || MODE == VARQ_GROUP_TENSOR;
    if (VIA_TOKENS)
        hipLaunchKernelGGL(group_clear_kernel, dim3(blocks((int64_t)a.B * a.L, 4096)), dim3(GQ_THREADS), 0, st,
                           a.packed, (int64_t)a.B, (int64_t)a.L, (int64_t)a.H * a.W * a.L_cap);
    else
        hipLaunchKernelGGL(group_clear_kernel, dim3(blocks(n_scales, 4096)), dim3(GQ_THREADS), 0, st,
                           a.absmax, (int64_t)1, n_scales, n_scales);
    hipLaunchKernelGGL(group_absmax_kernel<MODE>, dim3(blocks(n_items, grid_items)), dim3(GQ_THREADS), 0, st, a);
    if (VIA_TOKENS)
        hipLaunchKernelGGL(group_reduce_kernel<MODE>, dim3(MODE == VARQ_GROUP_BLOCK ? a.B * a.G : 1),
                           dim3(GQ_THREADS), 0, st, a);
    const float qmax = (float)((1 << (bits - 1)) - 1);
    hipLaunchKernelGGL(group_scale_kernel, dim3(blocks(n_scales, 4096)), dim3(GQ_THREADS), 0, st, a.absmax, n_scales, qmax);
    switch (bits) {
        case 2: hipLaunchKernelGGL((group_quant_kernel<2, MODE>), dim3(blocks(n_words, 1 << 20)), dim3(GQ_THREADS), 0, st, a); break;
        case 3: hipLaunchKernelGGL((group_quant_kernel<3, MODE>), dim3(blocks(n_words, 1 << 20)), dim3(GQ_THREADS), 0, st, a); break;
        case 4: hipLaunchKernelGGL((group_quant_kernel<4, MODE>), dim3(blocks(n_words, 1 << 20)), dim3(GQ_THREADS), 0, st, a); break;
        case 5: hipLaunchKernelGGL((group_quant_kernel<5, MODE>), dim3(blocks(n_words, 1 << 20)), dim3(GQ_THREADS), 0, st, a); break;
        case 6: hipLaunchKernelGGL((group_quant_kernel<6, MODE>), dim3(blocks(n_words, 1 << 20)), dim3(GQ_THREADS), 0, st, a); break;
        case 7: hipLaunchKernelGGL((group_quant_kernel<7, MODE>), dim3(blocks(n_words, 1 << 20)), dim3(GQ_THREADS), 0, st, a); break;
        case 8: hipLaunchKernelGGL((group_quant_kernel<8, MODE>), dim3(blocks(n_words, 1 << 20)), dim3(GQ_THREADS), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_group(const GroupArgs &a, int mode, int bits, int64_t n_scales, hipStream_t st) {
    switch (mode) {
        case VARQ_GROUP_BLOCK: return run_group<VARQ_GROUP_BLOCK>(a, bits, n_scales, 1 << 20, st);
        case VARQ_GROUP_TOKEN_HEAD: return run_group<VARQ_GROUP_TOKEN_HEAD>(a, bits, n_scales, 1 << 20, st);
        case VARQ_GROUP_TOKEN: return run_group<VARQ_GROUP_TOKEN>(a, bits, n_scales, 1 << 20, st);
        case VARQ_GROUP_TENSOR: return run_group<VARQ_GROUP_TENSOR>(a, bits, n_scales, 1 << 20, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace varq
