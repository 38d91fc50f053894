// quant_pack.hip - VAR-Q quantize+pack for gfx950.
//
// Project page (summary, "Next-block prediction", Fig. 8): one fp32 scale per
// (batch, head, generation block, channel), s = absmax / qmax; codes
// rint(x / s) packed LSB-first along head_dim into INT32 words.
//
// One work-group (256 threads, 4 waves) owns one unit = (batch, head, block,
// slice of whole words). Pass 1 streams the unit's bf16 rows once for the
// per-channel absmax (16-byte loads, lanes along the row); the partial maxima
// meet in LDS and give the slice's scales. Pass 2 streams the rows again,
// quantizes with the division-free exact quotient, stages the code fields in
// LDS and writes whole words, one word plane at a time, so that consecutive
// lanes store consecutive tokens of a plane.
#include "varq_device.h"

namespace varq {

constexpr int QP_THREADS = 256;

template <int BITS>
__global__ __launch_bounds__(QP_THREADS) void quant_pack_twopass(const QuantPackArgs a) {
    constexpr int CPW = 32 / BITS;
    constexpr uint32_t MASK = (1u << BITS) - 1u;
    constexpr float QMAX = (float)((1 << (BITS - 1)) - 1);

    __shared__ float red[QP_THREADS * 8];
    __shared__ float sh_s[256];
    __shared__ float sh_y[256];
    __shared__ uint8_t sh_codes[QP_THREADS * 12];   // rows x (slice channels + 4) code fields

    const int64_t unit = xcd_logical_id(blockIdx.x, a.n_units);
    if (unit < 0) return;

    // unit -> (block g, batch-head, slice): uniform binary search over unit_start
    int lo = 0, hi = a.G;                // unit_start[lo] <= unit < unit_start[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.unit_start[mid] <= unit) lo = mid; else hi = mid;
    }
    const int g = lo;
    const int sw = a.slice_words[g];
    const int n_slices = (a.W + sw - 1) / sw;
    const int64_t r_in_g = unit - a.unit_start[g];
    const int slice = (int)(r_in_g % n_slices);
    const int64_t bh = r_in_g / n_slices;
    const int b = (int)(bh / a.H), h = (int)(bh % a.H);

    const int w0 = slice * sw;
    const int c0 = w0 * CPW;
    const int c1 = min(a.D, (w0 + sw) * CPW);
    const int cs = c1 - c0;                 // multiple of 8 (host guarantees)
    const int ws = (cs + CPW - 1) / CPW;    // words in this slice
    const int lpr = cs >> 3;                // 16-byte chunks per row
    const int RP = QP_THREADS / lpr;        // rows per pass
    const int tid = threadIdx.x;
    const int chunk = tid % lpr, rr = tid / lpr;
    const bool active = rr < RP;

    const int64_t t0 = a.off[g];
    const int n = a.off[g + 1] - a.off[g];
    const uint16_t *xrow = a.x + (int64_t)b * a.sx_b + (int64_t)h * a.sx_h + c0 + 8 * chunk;

    // ---- pass 1: per-channel absmax
    float m[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) m[j] = 0.0f;
    if (active) {
        for (int r = rr; r < n; r += RP) {
            const uint4 v = *reinterpret_cast<const uint4 *>(xrow + (t0 + r) * a.sx_l);
            const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                m[2 * j] = fmaxf(m[2 * j], fabsf(bf16lo(wv[j])));
                m[2 * j + 1] = fmaxf(m[2 * j + 1], fabsf(bf16hi(wv[j])));
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) red[tid * 8 + j] = m[j];
    __syncthreads();
    if (tid < cs) {
        const int ch = tid >> 3, jj = tid & 7;
        float mx = 0.0f;
        for (int k = 0; k < RP; ++k) mx = fmaxf(mx, red[(k * lpr + ch) * 8 + jj]);
        const float s = mx / QMAX;                         // IEEE fp32 division
        sh_s[tid] = s;
        sh_y[tid] = recip_for_codes(s);
        a.scales[(((int64_t)b * a.H + h) * a.G_cap + a.group_start + g) * a.D + c0 + tid] = s;
    }
    __syncthreads();

    float s8[8], y8[8];
    bool fast = true;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        s8[j] = active ? sh_s[8 * chunk + j] : 0.0f;
        y8[j] = active ? sh_y[8 * chunk + j] : 0.0f;
        fast = fast && fast_scale_ok(s8[j]);
    }

    // ---- pass 2: codes -> LDS fields -> words
    const int pitch = cs + 4;
    uint32_t *plane0 = a.packed + (((int64_t)b * a.H + h) * a.W + w0) * a.L_cap + a.tok_start + t0;
    for (int base = 0; base < n; base += RP) {
        const int r = base + rr;
        if (active && r < n) {
            const uint4 v = *reinterpret_cast<const uint4 *>(xrow + (t0 + r) * a.sx_l);
            const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
            uint32_t f[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float xl = bf16lo(wv[j]), xh = bf16hi(wv[j]);
                int32_t ql, qh;
                if (fast) {
                    ql = code_fast(xl, s8[2 * j], y8[2 * j]);
                    qh = code_fast(xh, s8[2 * j + 1], y8[2 * j + 1]);
                } else {
                    ql = code_exact(xl, s8[2 * j]);
                    qh = code_exact(xh, s8[2 * j + 1]);
                }
                f[2 * j] = (uint32_t)ql & MASK;
                f[2 * j + 1] = (uint32_t)qh & MASK;
            }
            uint8_t *dst = sh_codes + rr * pitch + 8 * chunk;
            const uint32_t lo4 = f[0] | (f[1] << 8) | (f[2] << 16) | (f[3] << 24);
            const uint32_t hi4 = f[4] | (f[5] << 8) | (f[6] << 16) | (f[7] << 24);
            reinterpret_cast<uint32_t *>(dst)[0] = lo4;
            reinterpret_cast<uint32_t *>(dst)[1] = hi4;
        }
        __syncthreads();
        const int rows = min(RP, n - base);
        for (int i = tid; i < ws * rows; i += QP_THREADS) {
            const int wl = i / rows, rw = i % rows;
            const int cw0 = wl * CPW;
            const int ncodes = min(CPW, cs - cw0);
            const uint8_t *src = sh_codes + rw * pitch + cw0;
            uint32_t word = 0;
            for (int k = 0; k < ncodes; ++k) word |= (uint32_t)src[k] << (k * BITS);
            plane0[(int64_t)wl * a.L_cap + base + rw] = word;
        }
        __syncthreads();
    }
}

template <int BITS>
static hipError_t launch_qp(const QuantPackArgs &a, hipStream_t st) {
    const int64_t grid = ((int64_t)a.n_units + 7) / 8 * 8;
    hipLaunchKernelGGL(quant_pack_twopass<BITS>, dim3((unsigned)grid), dim3(QP_THREADS), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_quant_pack(const QuantPackArgs &a, int bits, hipStream_t st) {
    switch (bits) {
        case 2: return launch_qp<2>(a, st);
        case 3: return launch_qp<3>(a, st);
        case 4: return launch_qp<4>(a, st);
        case 5: return launch_qp<5>(a, st);
        case 6: return launch_qp<6>(a, st);
        case 7: return launch_qp<7>(a, st);
        case 8: return launch_qp<8>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace varq
