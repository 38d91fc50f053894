// packed_attention.hip - attention that reads the VAR-Q packed KV cache (gfx950).
//
// Project page "Next-block prediction": a block's queries attend to the cache of
// all earlier blocks and of itself, i.e. the window [0, L_kv) with no mask.
// README "Deployment Results" / "Memory-Efficient Runtime": loading the packed
// cache, unpacking and dequantizing are fused into attention.
//
// Work-group = 4 waves x 32 queries of one (batch, head). Per 64-token tile:
//  1. all 256 threads read packed words straight from HBM (each thread: one
//     word plane x 8 consecutive tokens = 32 bytes), dequantize them exactly to
//     bf16_rne(q * s[block(t), c]) and write K row-major (token x channel) and V
//     transposed (channel x token) into LDS;
//  2. each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (lanes hold
//     one query each, so the softmax row statistics are lane-local), runs an
//     online fp32 softmax in base 2, and accumulates O^T = V^T P^T with P kept in
//     registers: the accumulator layout of S^T is the B-operand layout of the PV
//     product up to a fixed permutation of the 16 tokens of a k-step, which the
//     V^T operand reads follow.
#include "varq_device.h"

namespace varq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int AT_THREADS = 256;
constexpr int AT_NT = 64;       // KV tokens per tile
constexpr int AT_QT = 128;      // queries per work-group (4 waves x 32)

__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int BITS, int D>
__global__ __launch_bounds__(AT_THREADS) void packed_attention_v1(const AttnArgs a) {
    constexpr int CPW = 32 / BITS;
    constexpr int W = (D + CPW - 1) / CPW;
    constexpr int SHIFT = 32 - BITS;
    constexpr int KP = D + 8;            // K row pitch (bf16)
    constexpr int VP = AT_NT + 8;        // V^T row pitch (bf16)
    constexpr int KSTEPS = D / 16;
    constexpr int DBLK = D / 32;

    __shared__ __attribute__((aligned(16))) uint16_t Ks[AT_NT * KP];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VP];
    __shared__ int32_t off[VARQ_MAX_GROUPS_DEV + 1];

    const int64_t n_blocks = (int64_t)a.n_qtiles * a.B * a.H;
    const int64_t lid = xcd_logical_id(blockIdx.x, n_blocks);
    if (lid < 0) return;
    const int qt = (int)(lid % a.n_qtiles);
    const int64_t bh = lid / a.n_qtiles;
    const int b = (int)(bh / a.H), h = (int)(bh % a.H);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 31, hf = lane >> 5;

    for (int i = tid; i <= a.G; i += AT_THREADS) off[i] = a.off[i];

    // Q^T operand: lane = query (lr), slots (hf, j) = channel 16*ks + 8*hf + j
    const int64_t qi = (int64_t)qt * AT_QT + wave * 32 + lr;
    const bool qvalid = qi < a.Lq;
    bf16x8 qop[KSTEPS];
    {
        const uint16_t *qrow = a.q + (int64_t)b * a.sq_b + qi * a.sq_l + (int64_t)h * a.sq_h + 8 * hf;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (qvalid) v = *reinterpret_cast<const uint4 *>(qrow + 16 * ks);
            qop[ks] = as_bf16x8(v);
        }
    }

    floatx16 o[DBLK];
#pragma unroll
    for (int d = 0; d < DBLK; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;

    const uint32_t *pk = a.pk + bh * W * a.L_cap;
    const uint32_t *pv = a.pv + bh * W * a.L_cap;
    const float *sk = a.sk + bh * a.G_cap * D;
    const float *sv = a.sv + bh * a.G_cap * D;
    int g_tile = 0;
    __syncthreads();

    for (int64_t n0 = 0; n0 < a.L_kv; n0 += AT_NT) {
        g_tile = group_of(off, g_tile, n0);
        __syncthreads();   // previous tile's LDS reads are done
        // ---- 1. load + unpack + dequant into LDS
        for (int it = tid; it < 16 * W; it += AT_THREADS) {
            const bool isV = it >= 8 * W;
            const int j = isV ? it - 8 * W : it;
            const int w = j >> 3, tg = j & 7;
            const int64_t t = n0 + 8 * tg;
            const uint32_t *plane = (isV ? pv : pk) + (int64_t)w * a.L_cap;
            uint32_t wd[8];
            if (t + 8 <= a.L_kv) {
                const uint4 v0 = *reinterpret_cast<const uint4 *>(plane + t);
                const uint4 v1 = *reinterpret_cast<const uint4 *>(plane + t + 4);
                wd[0] = v0.x; wd[1] = v0.y; wd[2] = v0.z; wd[3] = v0.w;
                wd[4] = v1.x; wd[5] = v1.y; wd[6] = v1.z; wd[7] = v1.w;
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) wd[k] = (t + k < a.L_kv) ? plane[t + k] : 0u;
            }
            const int cbase = w * CPW;
            const int ncw = min(CPW, D - cbase);
            const float *srow_base = isV ? sv : sk;
            int g = group_of(off, g_tile, t < a.L_kv ? t : a.L_kv - 1);
            float sc[CPW];
#pragma unroll
            for (int i = 0; i < CPW; ++i) sc[i] = (i < ncw) ? srow_base[(int64_t)g * D + cbase + i] : 0.0f;
            uint16_t vals[8][CPW];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int64_t tk = t + k;
                if (tk < a.L_kv && off[g + 1] <= tk) {
                    g = group_of(off, g, tk);
#pragma unroll
                    for (int i = 0; i < CPW; ++i)
                        sc[i] = (i < ncw) ? srow_base[(int64_t)g * D + cbase + i] : 0.0f;
                }
#pragma unroll
                for (int i = 0; i < CPW; ++i) {
                    const int32_t qv = (int32_t)(wd[k] << (SHIFT - i * BITS)) >> SHIFT;
                    vals[k][i] = (uint16_t)dequant_bits(qv, sc[i]);
                }
            }
            if (!isV) {
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    uint16_t *dst = Ks + (8 * tg + k) * KP + cbase;
                    if constexpr ((CPW * 2) % 16 == 0) {
#pragma unroll
                        for (int i = 0; i < CPW; i += 8) {
                            uint4 v;
                            v.x = vals[k][i] | ((uint32_t)vals[k][i + 1] << 16);
                            v.y = vals[k][i + 2] | ((uint32_t)vals[k][i + 3] << 16);
                            v.z = vals[k][i + 4] | ((uint32_t)vals[k][i + 5] << 16);
                            v.w = vals[k][i + 6] | ((uint32_t)vals[k][i + 7] << 16);
                            *reinterpret_cast<uint4 *>(dst + i) = v;
                        }
                    } else if constexpr ((CPW * 2) % 8 == 0) {
#pragma unroll
                        for (int i = 0; i < CPW; i += 4) {
                            uint2 v;
                            v.x = vals[k][i] | ((uint32_t)vals[k][i + 1] << 16);
                            v.y = vals[k][i + 2] | ((uint32_t)vals[k][i + 3] << 16);
                            *reinterpret_cast<uint2 *>(dst + i) = v;
                        }
                    } else if constexpr ((CPW * 2) % 4 == 0) {
#pragma unroll
                        for (int i = 0; i < CPW; i += 2)
                            if (i < ncw)
                                *reinterpret_cast<uint32_t *>(dst + i) =
                                    vals[k][i] | ((uint32_t)vals[k][i + 1] << 16);
                    } else {
#pragma unroll
                        for (int i = 0; i < CPW; ++i)
                            if (i < ncw) dst[i] = vals[k][i];
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < CPW; ++i) {
                    if (i < ncw) {
                        uint4 v;
                        v.x = vals[0][i] | ((uint32_t)vals[1][i] << 16);
                        v.y = vals[2][i] | ((uint32_t)vals[3][i] << 16);
                        v.z = vals[4][i] | ((uint32_t)vals[5][i] << 16);
                        v.w = vals[6][i] | ((uint32_t)vals[7][i] << 16);
                        *reinterpret_cast<uint4 *>(Vt + (cbase + i) * VP + 8 * tg) = v;
                    }
                }
            }
        }
        __syncthreads();

        // ---- 2. S^T = K Q^T for two 32-token blocks
        floatx16 s[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[tb][r] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const uint4 kv = *reinterpret_cast<const uint4 *>(Ks + (32 * tb + lr) * KP + 16 * ks + 8 * hf);
                s[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), qop[ks], s[tb], 0, 0, 0);
            }
        }
        // mask tokens past the window; tile max
        float mx = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t tok = n0 + 32 * tb + 8 * (r >> 2) + 4 * hf + (r & 3);
                if (tok >= a.L_kv) s[tb][r] = -INFINITY;
                mx = fmaxf(mx, s[tb][r]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx * a.scale_log2);
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < DBLK; ++d)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[d][r] *= alpha;

        bf16x8 pop[2][2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const float p = exp2f(__builtin_fmaf(s[tb][8 * hh + jj], a.scale_log2, -m_new));
                    l_run += p;
                    pop[tb][hh][jj] = (__bf16)p;
                }
            }
        }
        // ---- 3. O^T += V^T P^T
#pragma unroll
        for (int d = 0; d < DBLK; ++d) {
            const uint16_t *vrow = Vt + (32 * d + lr) * VP + 4 * hf;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int tk = 32 * tb + 16 * hh;
                    const uint2 lo = *reinterpret_cast<const uint2 *>(vrow + tk);
                    const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + tk + 8);
                    const uint4 av = make_uint4(lo.x, lo.y, hi.x, hi.y);
                    o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), pop[tb][hh], o[d], 0, 0, 0);
                }
            }
        }
    }

    // ---- normalise and store
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.0f / l_tot;
    if (qvalid) {
        uint16_t *orow = a.out + (int64_t)b * a.so_b + qi * a.so_l + (int64_t)h * a.so_h;
#pragma unroll
        for (int d = 0; d < DBLK; ++d) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int c = 32 * d + 8 * r4 + 4 * hf;
                uint2 v;
                v.x = bf16_bits_rne(o[d][4 * r4] * inv) | (bf16_bits_rne(o[d][4 * r4 + 1] * inv) << 16);
                v.y = bf16_bits_rne(o[d][4 * r4 + 2] * inv) | (bf16_bits_rne(o[d][4 * r4 + 3] * inv) << 16);
                *reinterpret_cast<uint2 *>(orow + c) = v;
            }
        }
    }
}

template <int BITS, int D>
static hipError_t launch_at(const AttnArgs &a, hipStream_t st) {
    const int64_t n_blocks = (int64_t)a.n_qtiles * a.B * a.H;
    const int64_t grid = (n_blocks + 7) / 8 * 8;
    hipLaunchKernelGGL((packed_attention_v1<BITS, D>), dim3((unsigned)grid), dim3(AT_THREADS), 0, st, a);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_at_bits(const AttnArgs &a, int bits, hipStream_t st) {
    switch (bits) {
        case 2: return launch_at<2, D>(a, st);
        case 3: return launch_at<3, D>(a, st);
        case 4: return launch_at<4, D>(a, st);
        case 5: return launch_at<5, D>(a, st);
        case 6: return launch_at<6, D>(a, st);
        case 7: return launch_at<7, D>(a, st);
        case 8: return launch_at<8, D>(a, st);
        default: return hipErrorInvalidValue;
    }
}

int attention_q_tile() { return AT_QT; }

hipError_t launch_packed_attention(const AttnArgs &a, int D, int bits, hipStream_t st) {
    if (D == 64) return launch_at_bits<64>(a, bits, st);
    if (D == 128) return launch_at_bits<128>(a, bits, st);
    return hipErrorInvalidValue;
}

}  // namespace varq
