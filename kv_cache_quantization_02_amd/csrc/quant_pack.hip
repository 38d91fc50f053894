// quant_pack.hip - VAR-Q quantize+pack for gfx950, one read of the input.
//
// Project page (summary, "Next-block prediction", Fig. 8): one fp32 scale per
// (batch, head, generation block, channel), s = absmax / qmax; codes
// rint(x / s) packed LSB-first along head_dim into INT32 words.
//
// Work unit = up to T token rows of one (batch, head), T * D = 16384 elements:
// either one chunk of a block longer than T, or a pack of up to QP_MAX_PACK
// whole consecutive blocks. A 256-thread work-group loads a unit into registers
// once (16-byte loads, lanes along a row) and takes the per-(block, channel)
// absmax: packed 16-bit maxima of |x| bit patterns in registers, then LDS
// max-atomics. It quantizes from registers with the division-free exact
// quotient and writes whole words: at 2, 4, 7 and 8 bits a lane's 8 channels
// (a lane pair's 16 at 2 bits) form whole words directly; at 3, 5 and 6 bits
// the fields are staged in LDS and stored plane by plane. Either way the lanes
// of a work-group cover every token of the unit in each word plane.
//
// A block split over several chunks needs the maximum over all of them. Every
// chunk but the last publishes its partial maxima in a scratch slot tagged with
// this launch's epoch; the last chunk gathers them (waiting on each tag),
// publishes the block maximum the same way and quantizes at once. The other
// chunks defer their quantization: a work-group keeps the waiting unit in a
// second register set, processes its next unit, and only then waits for the
// block maximum. Each value crosses work-groups in one 64-bit atomic word that
// carries both the tag and the maximum, so no cache flush or fence is needed
// for it; the epoch advances once per launch, set by the last work-group to
// finish.
//
// Progress for the waits (such launches are cooperative: every work-group is
// resident). Work-group w takes units w, w + grid, ...; for each unit u it
// publishes P(u) (partial, or block maximum for a last chunk), then finishes
// F(u') of the unit it deferred one step earlier. Let x be the smallest unit
// whose P never happens. Before P(x) its work-group needs P(x - grid) and
// F(x - 2 grid); the latter needs P of the last chunk of that unit's block,
// which is < x when no block has more than grid chunks; and if x is a last
// chunk it needs P of the earlier chunks of its block, all < x. So P(x)
// happens, a contradiction; every F(u) then follows. Spins are nevertheless
// bounded and report a timeout through a status word.
#include "varq_device.h"

namespace varq {

constexpr int QP_THREADS = 256;
constexpr int QP_ITEMS = 8;                                  // 16-byte row chunks held per thread
constexpr int QP_UNIT_ELEMS = QP_THREADS * QP_ITEMS * 8;     // 16384 elements per unit
constexpr int QP_MAX_PACK = 8;                               // blocks per packed unit
constexpr int QP_SLOT_Y = QP_MAX_PACK;                       // scale slot of the deferred unit
constexpr unsigned QP_SPIN_LIMIT = 1u << 22;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Wave-uniform description of a unit.
struct Unit {
    int64_t id, bh;
    int g0, nb;          // first block, number of blocks (> 1 only for packs)
    int c, nc;           // chunk index and chunk count of block g0 (nc == 1 for packs)
    int row0, n;         // first row relative to x, rows
};

__device__ inline Unit unit_of(const QuantPackArgs &a, int64_t id) {
    Unit U;
    U.id = id;
    U.bh = id / a.units_per_bh;
    const int r_in = (int)(id - U.bh * a.units_per_bh);
    int lo = 0, hi = a.G;                 // last g with unit_start[g] <= r_in
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.unit_start[mid] <= r_in) lo = mid; else hi = mid;
    }
    const int T = a.chunk_rows;
    const int len = a.off[lo + 1] - a.off[lo];
    if (len > T) {
        U.g0 = lo; U.nb = 1;
        U.c = r_in - a.unit_start[lo];
        U.nc = (len + T - 1) / T;
        U.row0 = a.off[lo] + U.c * T;
        U.n = min(T, a.off[lo + 1] - U.row0);
    } else {
        int g0 = lo;
        while (g0 > 0 && a.unit_start[g0 - 1] == r_in) --g0;
        U.g0 = g0; U.nb = lo - g0 + 1;
        U.c = 0; U.nc = 1;
        U.row0 = a.off[g0];
        U.n = a.off[lo + 1] - a.off[g0];
    }
    return U;
}

// Local block (0 .. nb-1) of unit row r.
__device__ inline int local_block(const QuantPackArgs &a, const Unit &U, int r) {
    int lb = 0;
    const int t = U.row0 + r;
    for (int j = 1; j < U.nb; ++j) lb += t >= a.off[U.g0 + j] ? 1 : 0;
    return lb;
}

struct Lane {
    int chunk, rr, RP, lpr;
    bool active;
};

// Issue the 16-byte row-chunk loads of unit U into v (all in flight at once).
__device__ inline void load_unit(const QuantPackArgs &a, const Unit &U, uint4 (&v)[QP_ITEMS], const Lane &L) {
    const int64_t b = U.bh / a.H, h = U.bh - b * a.H;
    const uint16_t *xbase = a.x + b * a.sx_b + h * a.sx_h + 8 * L.chunk + (int64_t)U.row0 * a.sx_l;
#pragma unroll
    for (int k = 0; k < QP_ITEMS; ++k) {
        const int r = L.rr + k * L.RP;
        v[k] = make_uint4(0, 0, 0, 0);
        if (L.active && r < U.n) v[k] = *reinterpret_cast<const uint4 *>(xbase + (int64_t)r * a.sx_l);
    }
}

__device__ inline void flush_max(uint32_t *sh_max, int lb, int chunk, const u16x2 (&m)[4]) {
    uint32_t *dst = sh_max + lb * 256 + 8 * chunk;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t w = __builtin_bit_cast(uint32_t, m[j]);
        atomicMax(dst + 2 * j, w << 16);
        atomicMax(dst + 2 * j + 1, w & 0xFFFF0000u);
    }
}

__device__ inline void absmax_item(u16x2 (&m)[4], const uint4 &w) {
    const u16x2 mask = u16x2{0x7FFF, 0x7FFF};
    m[0] = __builtin_elementwise_max(m[0], __builtin_bit_cast(u16x2, w.x) & mask);
    m[1] = __builtin_elementwise_max(m[1], __builtin_bit_cast(u16x2, w.y) & mask);
    m[2] = __builtin_elementwise_max(m[2], __builtin_bit_cast(u16x2, w.z) & mask);
    m[3] = __builtin_elementwise_max(m[3], __builtin_bit_cast(u16x2, w.w) & mask);
}

// Per-(local block, channel) absmax of the unit in v, merged into sh_max as
// fp32 bit patterns (non-negative floats order like their bit patterns; the
// bf16 bit pattern of |x| is that of x with the sign bit cleared).
__device__ inline void unit_absmax(const QuantPackArgs &a, const Unit &U, const uint4 (&v)[QP_ITEMS],
                                   const Lane &L, uint32_t *sh_max) {
    if (!L.active) return;
    u16x2 m[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = u16x2{0, 0};
    if (U.nb == 1) {
#pragma unroll
        for (int k = 0; k < QP_ITEMS; ++k) absmax_item(m, v[k]);      // rows past n hold zeros
        flush_max(sh_max, 0, L.chunk, m);
        return;
    }
    int cur = 0;
#pragma unroll
    for (int k = 0; k < QP_ITEMS; ++k) {
        const int r = L.rr + k * L.RP;
        if (r < U.n) {
            const int lb = local_block(a, U, r);          // non-decreasing in k
            if (lb != cur) {
                flush_max(sh_max, cur, L.chunk, m);
#pragma unroll
                for (int j = 0; j < 4; ++j) m[j] = u16x2{0, 0};
                cur = lb;
            }
            absmax_item(m, v[k]);
        }
    }
    flush_max(sh_max, cur, L.chunk, m);
}

// b-bit two's complement fields (low bits of each word, higher bits garbage)
// of the 8 channels in w under scales s8 and reciprocals y8.
__device__ inline void codes8(const uint4 &w, const float (&s8)[8], const float (&y8)[8], bool fast,
                              uint32_t (&f)[8]) {
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float xl = bf16lo(wv[j]), xh = bf16hi(wv[j]);
        if (fast) {
            f[2 * j] = (uint32_t)code_fast(xl, s8[2 * j], y8[2 * j]);
            f[2 * j + 1] = (uint32_t)code_fast(xh, s8[2 * j + 1], y8[2 * j + 1]);
        } else {
            f[2 * j] = (uint32_t)code_exact(xl, s8[2 * j]);
            f[2 * j + 1] = (uint32_t)code_exact(xh, s8[2 * j + 1]);
        }
    }
}

__device__ inline void load_sy(const float *sh_s, const float *sh_y, int slot, int chunk, float (&s8)[8],
                               float (&y8)[8], bool &fast) {
    const float4 *ps = reinterpret_cast<const float4 *>(sh_s + slot * 256 + 8 * chunk);
    const float4 *py = reinterpret_cast<const float4 *>(sh_y + slot * 256 + 8 * chunk);
    const float4 s0 = ps[0], s1 = ps[1], y0 = py[0], y1 = py[1];
    s8[0] = s0.x; s8[1] = s0.y; s8[2] = s0.z; s8[3] = s0.w;
    s8[4] = s1.x; s8[5] = s1.y; s8[6] = s1.z; s8[7] = s1.w;
    y8[0] = y0.x; y8[1] = y0.y; y8[2] = y0.z; y8[3] = y0.w;
    y8[4] = y1.x; y8[5] = y1.y; y8[6] = y1.z; y8[7] = y1.w;
    fast = true;
#pragma unroll
    for (int j = 0; j < 8; ++j) fast = fast && fast_scale_ok(s8[j]);
}

// Quantize and store unit U (rows in v) with the scales of LDS slot `slot`
// (packs: slot = local block). Ends with a barrier, after which LDS may be
// rewritten.
template <int BITS>
__device__ inline void quantize_unit(const QuantPackArgs &a, const Unit &U, const uint4 (&v)[QP_ITEMS],
                                     const Lane &L, int slot, const float *sh_s, const float *sh_y,
                                     uint8_t *sh_codes) {
    constexpr int CPW = 32 / BITS;
    constexpr uint32_t MASK = (1u << BITS) - 1u;
    const int tid = threadIdx.x;
    const int D = a.D;
    uint32_t *plane0 = a.packed + U.bh * a.W * a.L_cap + a.tok_start + U.row0;
    // a 2-bit word takes a lane pair (16 channels); with an odd lane count per
    // row the last chunk has no partner, so that case is staged in LDS like
    // 3, 5 and 6 bits
    const bool direct = (BITS == 4 || BITS == 7 || BITS == 8) || (BITS == 2 && (L.lpr & 1) == 0);

    float s8[8], y8[8];
    bool fast = true;
    int cur = -1;
    if (U.nb == 1 && L.active) { load_sy(sh_s, sh_y, slot, L.chunk, s8, y8, fast); cur = slot; }

    if (direct) {
#pragma unroll
        for (int k = 0; k < QP_ITEMS; ++k) {
            const int r = L.rr + k * L.RP;
            const bool live = L.active && r < U.n;
            uint32_t f[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) f[j] = 0;
            if (live) {
                if (U.nb > 1) {
                    const int lb = local_block(a, U, r);
                    if (lb != cur) { load_sy(sh_s, sh_y, lb, L.chunk, s8, y8, fast); cur = lb; }
                }
                codes8(v[k], s8, y8, fast, f);
            }
            if constexpr (BITS == 4) {
                uint32_t w = 0;
#pragma unroll
                for (int j = 0; j < 8; ++j) w |= (f[j] & MASK) << (4 * j);
                if (live) plane0[(int64_t)L.chunk * a.L_cap + r] = w;
            } else if constexpr (BITS == 7 || BITS == 8) {
                uint32_t w0 = 0, w1 = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    w0 |= (f[j] & MASK) << (BITS * j);
                    w1 |= (f[4 + j] & MASK) << (BITS * j);
                }
                if (live) {
                    plane0[(int64_t)(2 * L.chunk) * a.L_cap + r] = w0;
                    plane0[(int64_t)(2 * L.chunk + 1) * a.L_cap + r] = w1;
                }
            } else if constexpr (BITS == 2) {
                uint32_t half = 0;
#pragma unroll
                for (int j = 0; j < 8; ++j) half |= (f[j] & MASK) << (2 * j);
                // chunk ^ 1 of the same row: lane tid ^ 1 (rows hold an even number of lanes)
                const uint32_t other = (uint32_t)__shfl_xor((int)half, 1);
                if (live && (L.chunk & 1) == 0) plane0[(int64_t)(L.chunk >> 1) * a.L_cap + r] = half | (other << 16);
            }
        }
        __syncthreads();
        return;
    }

    // ---- fields -> LDS code rows -> words, one plane at a time
    const int pitch = D >= 64 ? D + 4 : D;
#pragma unroll
    for (int k = 0; k < QP_ITEMS; ++k) {
        const int r = L.rr + k * L.RP;
        if (L.active && r < U.n) {
            if (U.nb > 1) {
                const int lb = local_block(a, U, r);
                if (lb != cur) { load_sy(sh_s, sh_y, lb, L.chunk, s8, y8, fast); cur = lb; }
            }
            uint32_t f[8];
            codes8(v[k], s8, y8, fast, f);
            uint8_t *dst = sh_codes + r * pitch + 8 * L.chunk;
            *reinterpret_cast<uint32_t *>(dst) =
                (f[0] & MASK) | ((f[1] & MASK) << 8) | ((f[2] & MASK) << 16) | ((f[3] & MASK) << 24);
            *reinterpret_cast<uint32_t *>(dst + 4) =
                (f[4] & MASK) | ((f[5] & MASK) << 8) | ((f[6] & MASK) << 16) | ((f[7] & MASK) << 24);
        }
    }
    __syncthreads();
    const int tshift = a.rows_log2;
    const int span = 1 << tshift;
    for (int i = tid; i < a.W * span; i += QP_THREADS) {
        const int w = i >> tshift, r = i & (span - 1);
        if (r >= U.n) continue;
        const int cw0 = w * CPW;
        const uint8_t *src = sh_codes + r * pitch + cw0;
        uint32_t word = 0;
        if (cw0 + CPW <= D) {
#pragma unroll
            for (int q = 0; q < CPW; ++q) word |= (uint32_t)src[q] << (q * BITS);
        } else {
            for (int q = 0; q < D - cw0; ++q) word |= (uint32_t)src[q] << (q * BITS);
        }
        plane0[(int64_t)w * a.L_cap + r] = word;
    }
    __syncthreads();
}

__device__ inline uint64_t tagged(uint32_t epoch, float m) { return ((uint64_t)epoch << 32) | f2u(m); }

// Wait until the 64-bit slot carries `epoch`; returns the maximum it holds.
__device__ inline float wait_slot(const uint64_t *p, uint32_t epoch, uint32_t *status) {
    unsigned spins = 0;
    uint64_t v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while ((uint32_t)(v >> 32) != epoch) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > QP_SPIN_LIMIT) {
            __hip_atomic_store(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return u2f((uint32_t)v);
}

template <int BITS>
__global__ __launch_bounds__(QP_THREADS) void quant_pack_onepass(const QuantPackArgs a) {
    constexpr float QMAX = (float)((1 << (BITS - 1)) - 1);
    __shared__ __attribute__((aligned(16))) uint32_t sh_max[QP_MAX_PACK * 256];
    __shared__ __attribute__((aligned(16))) float sh_s[(QP_MAX_PACK + 1) * 256];
    __shared__ __attribute__((aligned(16))) float sh_y[(QP_MAX_PACK + 1) * 256];
    __shared__ __attribute__((aligned(16))) uint8_t sh_codes[QP_UNIT_ELEMS + 4 * 512];

    const int tid = threadIdx.x;
    const int D = a.D;
    Lane L;
    L.lpr = D >> 3;
    L.RP = QP_THREADS / L.lpr;
    L.chunk = tid % L.lpr;
    L.rr = tid / L.lpr;
    L.active = L.rr < L.RP;
    const int64_t step = gridDim.x;
    const bool split = a.part != nullptr;     // some block spans several chunks

    uint32_t epoch = 0;
    if (split) {
        epoch = __hip_atomic_load(a.sync, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) + 1u;
        if (epoch == 0) epoch = 1;
    }
    for (int i = tid; i < QP_MAX_PACK * 256; i += QP_THREADS) sh_max[i] = 0;
    __syncthreads();

    uint4 X[QP_ITEMS], Y[QP_ITEMS], Z[QP_ITEMS];
    Unit UX, UY, UZ;
    bool pendY = false;
    int64_t u = blockIdx.x;
    if (u < a.n_units) { UZ = unit_of(a, u); load_unit(a, UZ, Z, L); }
    while (u < a.n_units) {
        UX = UZ;
#pragma unroll
        for (int k = 0; k < QP_ITEMS; ++k) X[k] = Z[k];
        u += step;
        if (u < a.n_units) { UZ = unit_of(a, u); load_unit(a, UZ, Z, L); }

        // ---- absmax of X; a split block's chunks exchange maxima
        unit_absmax(a, UX, X, L, sh_max);
        __syncthreads();
        const bool deferX = UX.nc > 1 && UX.c < UX.nc - 1;
        float m0 = 0.0f;
        if (tid < D) {
            m0 = u2f(sh_max[tid]);
            if (UX.nc > 1) {
                if (deferX) {
                    __hip_atomic_store(a.part + UX.id * D + tid, tagged(epoch, m0), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                } else {
                    for (int cc = 0; cc < UX.nc - 1; ++cc)
                        m0 = fmaxf(m0, wait_slot(a.part + (UX.id - UX.c + cc) * D + tid, epoch, a.sync + 2));
                    __hip_atomic_store(a.fin + (UX.bh * a.G + UX.g0) * D + tid, tagged(epoch, m0),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }

        // ---- scales: the deferred unit Y (block maximum from its last chunk),
        // and X unless X waits now; the block maxima in LDS are cleared for the
        // next unit (the barrier below orders that before its max-atomics)
        if (tid < D) {
            if (pendY) {
                const float m = wait_slot(a.fin + (UY.bh * a.G + UY.g0) * D + tid, epoch, a.sync + 2);
                const float s = m / QMAX;                            // IEEE fp32 division
                sh_s[QP_SLOT_Y * 256 + tid] = s;
                sh_y[QP_SLOT_Y * 256 + tid] = recip_for_codes(s);
            }
            sh_max[tid] = 0;
            if (!deferX) {
                float *scl = a.scales + (UX.bh * a.G_cap + a.group_start + UX.g0) * D + tid;
                for (int lb = 0; lb < UX.nb; ++lb) {
                    float m = m0;
                    if (lb > 0) {
                        m = u2f(sh_max[lb * 256 + tid]);
                        sh_max[lb * 256 + tid] = 0;
                    }
                    const float s = m / QMAX;                        // IEEE fp32 division
                    sh_s[lb * 256 + tid] = s;
                    sh_y[lb * 256 + tid] = recip_for_codes(s);
                    scl[(int64_t)lb * D] = s;
                }
            }
        }
        __syncthreads();
        if (pendY) quantize_unit<BITS>(a, UY, Y, L, QP_SLOT_Y, sh_s, sh_y, sh_codes);
        if (!deferX) {
            quantize_unit<BITS>(a, UX, X, L, 0, sh_s, sh_y, sh_codes);
            pendY = false;
        } else {
            UY = UX;
#pragma unroll
            for (int k = 0; k < QP_ITEMS; ++k) Y[k] = X[k];
            pendY = true;
        }
    }
    if (pendY) {
        if (tid < D) {
            const float m = wait_slot(a.fin + (UY.bh * a.G + UY.g0) * D + tid, epoch, a.sync + 2);
            const float s = m / QMAX;
            sh_s[QP_SLOT_Y * 256 + tid] = s;
            sh_y[QP_SLOT_Y * 256 + tid] = recip_for_codes(s);
        }
        __syncthreads();
        quantize_unit<BITS>(a, UY, Y, L, QP_SLOT_Y, sh_s, sh_y, sh_codes);
    }

    // ---- the last work-group to finish advances the epoch for the next launch
    if (split && tid == 0) {
        const uint32_t done = __hip_atomic_fetch_add(a.sync + 1, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {
            __hip_atomic_store(a.sync + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.sync, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int BITS>
static hipError_t launch_qp(const QuantPackArgs &a, int grid, bool cooperative, hipStream_t st) {
    if (!cooperative) {
        hipLaunchKernelGGL(quant_pack_onepass<BITS>, dim3(grid), dim3(QP_THREADS), 0, st, a);
        return hipGetLastError();
    }
    void *args[] = {const_cast<QuantPackArgs *>(&a)};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void *>(&quant_pack_onepass<BITS>),
                                      dim3(grid), dim3(QP_THREADS), args, 0, st);
}

template <int BITS>
static int qp_resident_blocks() {
    int per_cu = 0, cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quant_pack_onepass<BITS>, QP_THREADS, 0) != hipSuccess)
        return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return per_cu * cus;
}

int quant_pack_unit_elems() { return QP_UNIT_ELEMS; }
int quant_pack_max_pack() { return QP_MAX_PACK; }

int quant_pack_resident_blocks(int bits) {
    constexpr int kMaxDev = 64;
    static int cached[kMaxDev][9];   // resident work-groups per (device, bits); 0 = not yet queried
    int dev = 0;
    if (bits < 2 || bits > 8 || hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev < kMaxDev && cached[dev][bits] > 0) return cached[dev][bits];
    int r = 0;
    switch (bits) {
        case 2: r = qp_resident_blocks<2>(); break;
        case 3: r = qp_resident_blocks<3>(); break;
        case 4: r = qp_resident_blocks<4>(); break;
        case 5: r = qp_resident_blocks<5>(); break;
        case 6: r = qp_resident_blocks<6>(); break;
        case 7: r = qp_resident_blocks<7>(); break;
        case 8: r = qp_resident_blocks<8>(); break;
    }
    if (dev < kMaxDev) cached[dev][bits] = r;
    return r;
}

hipError_t launch_quant_pack(const QuantPackArgs &a, int bits, int grid, bool cooperative, hipStream_t st) {
    switch (bits) {
        case 2: return launch_qp<2>(a, grid, cooperative, st);
        case 3: return launch_qp<3>(a, grid, cooperative, st);
        case 4: return launch_qp<4>(a, grid, cooperative, st);
        case 5: return launch_qp<5>(a, grid, cooperative, st);
        case 6: return launch_qp<6>(a, grid, cooperative, st);
        case 7: return launch_qp<7>(a, grid, cooperative, st);
        case 8: return launch_qp<8>(a, grid, cooperative, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace varq
