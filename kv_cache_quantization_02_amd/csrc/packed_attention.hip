// packed_attention.hip - attention that reads the VAR-Q packed KV cache (gfx950).
//
// Project page "Next-block prediction": a block's queries attend to the cache of
// all earlier blocks and of itself, i.e. the window [0, L_kv) with no mask.
// README "Deployment Results" / "Memory-Efficient Runtime": loading the packed
// cache, unpacking and dequantizing are fused into attention.
//
// Work-group = 8 waves x 32 queries of one (batch, head) and one range of the
// KV tiles (the whole window unless the grid is too small to fill the device;
// then the ranges' partial results are merged by merge_kv_splits). Tiles of 64
// tokens are software pipelined with one LDS barrier per tile:
//  * the packed words of tile j+2 are fetched into registers (an item = 4
//    consecutive tokens of one word plane = one 16-byte load per thread);
//  * tile j is consumed by each wave: S^T = K Q^T with v_mfma_f32_32x32x16_bf16
//    (a lane owns one query, so softmax statistics are lane-local), base-2
//    softmax in fp32 against a running maximum that is raised only when a
//    half-tile's exponentials leave [0, 2^64), and O^T += V^T P^T with P taken
//    straight from the S^T accumulators (their layout is the B-operand layout
//    of the PV product up to a fixed permutation of each 16-token k-step, which
//    the V^T layout follows). Row sums use v_dot2 on the bf16 P actually
//    multiplied. The second half's score MFMAs are interleaved with the first
//    half's exponentials, and the first half's P*V with the second half's
//    exponentials: the matrix core and the vector ALUs overlap only when their
//    instructions alternate within one wave;
//  * tile j+1 is then dequantized exactly, bf16_rne(q * s[block(t), c]), from
//    the registers into the free half of the double-buffered LDS - K row-major
//    (token x channel), V transposed (channel x token).
// Only the last tile of the window masks tokens past it; only tiles that
// contain a block boundary take the per-token scale path.
#include "varq_device.h"
#include "varq_tile_math.h"

#include <type_traits>
#include <utility>

namespace varq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int AT_NT = 64;        // KV tokens per tile
// LDS operand reads run this many matrix steps ahead of their use in the
// interleaved phases of a tile
constexpr int AT_RA = 2;
// blocks whose K and V scales a work-group holds in LDS: at head_dim 64 two
// work-groups still share a CU's LDS, at 128 (one work-group per CU) the
// scales of 64 blocks take 64 KB next to the 72 KB of tile buffers
template <int D>
constexpr int at_sl_maxg() { return D == 64 ? 32 : 64; }

__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ inline bf16x2 ones_bf16x2() {
    return __builtin_bit_cast(bf16x2, 0x3F803F80u);
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
    floatx2 f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

template <int BITS>
__device__ inline float field_f32(uint32_t word, int i) {
    constexpr int SHIFT = 32 - BITS;
    return (float)((int32_t)(word << (SHIFT - i * BITS)) >> SHIFT);
}

// (float)(int8_t)(byte J of x): one SDWA conversion of a sign-extended byte
template <int J>
__device__ inline float sbyte_f32(uint32_t x) {
    float r;
    if constexpr (J == 0)
        asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(r) : "v"(x));
    else if constexpr (J == 1)
        asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(x));
    else if constexpr (J == 2)
        asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(x));
    else
        asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(x));
    return r;
}

// Byte decode of INT4 and INT8 words: field i of an INT8 word is byte i; the
// fields 2j, 2j + 1 of an INT4 word are byte j of (w << 4) & 0xF0F0F0F0 and of
// w & 0xF0F0F0F0, each the code times 16 as a signed byte. Codes (times 16)
// then take the scale (over 16) from the LDS table: the product, and its one
// rounding, equal fp32(q) * s wherever s / 16 is exact.
template <int BITS>
struct ByteWord {
    static_assert(BITS == 4 || BITS == 8, "byte decode");
    uint32_t lo, hi;
    __device__ explicit ByteWord(uint32_t w) {
        if constexpr (BITS == 4) { lo = (w << 4) & 0xF0F0F0F0u; hi = w & 0xF0F0F0F0u; }
        else { lo = w; hi = 0; }
    }
    // field I as a float: 16 q (INT4) or q (INT8)
    template <int I>
    __device__ float field() const {
        if constexpr (BITS == 4) return sbyte_f32<I / 2>((I & 1) ? hi : lo);
        else return sbyte_f32<I>(lo);
    }
};

template <typename F, int... I>
__device__ inline void static_for_impl(F &f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>)
template <int N, typename F>
__device__ inline void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// o *= alpha on an accumulator tile
__device__ inline void scale_acc16(floatx16 &o, float alpha) {
#pragma unroll
    for (int r = 0; r < 16; ++r) o[r] *= alpha;
}

// BITS = 16 (DENSE): K and V are plain bf16 [B, H, rows, D] (the unfused
// baseline: unpack+dequant first, then this kernel); items are then 4 tokens
// x 8 channels of K or V.
template <int BITS, int D, int QB, int NW>
struct AttnTile {
    static constexpr bool DENSE = BITS == 16;
    static constexpr int CPW = DENSE ? 8 : 32 / BITS;
    static constexpr int W = (D + CPW - 1) / CPW;
    static constexpr int KP = D + 8;          // K row pitch (bf16)
    static constexpr int VP = AT_NT + 8;      // V^T row pitch (bf16)
    static constexpr int THREADS = 64 * NW;
    static constexpr int QW = 32 * QB;        // queries per wave
    static constexpr int QT = NW * QW;        // queries per work-group
    // 16W K items (4 tokens of one word plane each), then 16W V items. The K
    // items' slots are padded to whole waves, so every wave holds items of one
    // kind (or none) at each of its IPT positions.
    static constexpr int NK = 16 * W;
    static constexpr int NKP = (NK + 63) / 64 * 64;
    static constexpr int NSLOTS = NKP + NK;
    static constexpr int WORDS = DENSE ? 16 : 4;   // 32-bit words an item loads
    static constexpr int IPT = (NSLOTS + THREADS - 1) / THREADS;
};

// V^T tile in LDS: row = channel; inside each 16-token group the four 4-token
// quarters are stored in the order 0, 2, 1, 3 so that the eight tokens one PV
// operand lane needs (quarters hf and hf + 2) are contiguous.
__device__ inline int v_pos(int tok) {
    const int q = (tok >> 2) & 3;
    return (tok & ~15) + 4 * (((q & 1) << 1) | (q >> 1)) + (tok & 3);
}

// SL: the (batch, head)'s K and V scales (at most at_sl_maxg<D>() blocks) are
// copied to LDS once, and dequantization reads them there; otherwise each
// tile's scales are prefetched from memory with its words.
// ROPE (pre-RoPE quantization, project page Appendix F / Table 7): K was
// quantized before the rotary embedding; every dequantized K tile is rotated
// in LDS, pair (2i, 2i+1) of token t by cos/sin[t, i] (fp32, each product and
// the sum rounded, then bf16), before the scores use it.
template <int BITS, int D, int QB, int NW, bool SL, bool ROPE = false>
__global__ __launch_bounds__(64 * NW) void packed_attention_v5(const AttnArgs a) {
    using T = AttnTile<BITS, D, QB, NW>;
    constexpr bool DENSE = T::DENSE;
    constexpr int CPW = T::CPW, W = T::W, KP = T::KP, VP = T::VP;
    constexpr int THREADS = T::THREADS, QW = T::QW, QT = T::QT;
    constexpr int NKP = T::NKP, NSLOTS = T::NSLOTS, IPT = T::IPT;
    constexpr int KSTEPS = D / 16;
    constexpr int DBLK = D / 32;
    constexpr int KBUF = AT_NT * KP, VBUF = D * VP;

    __shared__ __attribute__((aligned(16))) uint16_t Ks[2 * KBUF];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[2 * VBUF];
    __shared__ int32_t off[VARQ_MAX_GROUPS_DEV + 1];
    constexpr int SLG = at_sl_maxg<D>();
    __shared__ __attribute__((aligned(16))) float sS[SL ? 2 * SLG * D : 4];   // K rows, then V rows

    const int n_blocks = a.n_qtiles * a.B * a.H * a.kv_splits;
    const int lid = (int)xcd_logical_id(blockIdx.x, n_blocks);
    if (lid < 0) return;
    // logical id = ((b*H + h) * kv_splits + split) * n_qtiles + q-tile: the
    // q-tiles of one KV range run on one XCD and share its L2
    const int qt = lid % a.n_qtiles;
    const int split = (lid / a.n_qtiles) % a.kv_splits;
    const int bh = lid / a.n_qtiles / a.kv_splits;
    const int b = bh / a.H, h = bh % a.H;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 31, hf = lane >> 5;

    for (int i = tid; i <= a.G; i += THREADS) off[i] = a.off[i];
    // INT4 with scales in LDS: when every scale over 16 is exact, the table
    // holds s / 16 for the byte decode (ByteWord); otherwise s
    bool byte16 = false;
    auto div16_exact = [](float4 v) {
        auto ok1 = [](float x) { return x == 0.0f || x >= 0x1p-122f; };
        return ok1(v.x) && ok1(v.y) && ok1(v.z) && ok1(v.w);
    };
    auto over16 = [](float4 v) { return make_float4(v.x * 0.0625f, v.y * 0.0625f, v.z * 0.0625f, v.w * 0.0625f); };
    // scales kept in LDS: up to SLP float4 of K and as many of V per thread.
    // With one of each they are loaded now and stored once the loads below
    // have all been waited for; with more they are copied first, before any
    // other load is in flight, so that no register holds them for long.
    constexpr int SLP = SL ? (SLG * D / 4 + THREADS - 1) / THREADS : 1;
    float4 sl_k = make_float4(0.f, 0.f, 0.f, 0.f), sl_v = sl_k;
    if constexpr (SL) {
        const float4 *gk = reinterpret_cast<const float4 *>(a.sk + (int64_t)bh * a.G_cap * D);
        const float4 *gv = reinterpret_cast<const float4 *>(a.sv + (int64_t)bh * a.G_cap * D);
        if constexpr (SLP == 1) {
            if (tid < a.G * (D / 4)) {
                sl_k = gk[tid];
                sl_v = gv[tid];
            }
        } else {
            // loads past the scales re-read the last vector (not stored)
            const int n4 = a.G * (D / 4);
            float4 ck[SLP], cv[SLP];
#pragma unroll
            for (int i = 0; i < SLP; ++i) {
                const int e = min(tid + THREADS * i, n4 - 1);
                ck[i] = gk[e];
                cv[i] = gv[e];
            }
            bool ok = true;
#pragma unroll
            for (int i = 0; i < SLP; ++i) ok = ok && div16_exact(ck[i]) && div16_exact(cv[i]);
            byte16 = BITS == 4 && __syncthreads_and(ok ? 1 : 0) != 0;
#pragma unroll
            for (int i = 0; i < SLP; ++i) {
                const int e = tid + THREADS * i;
                if (e < n4) {
                    reinterpret_cast<float4 *>(sS)[e] = byte16 ? over16(ck[i]) : ck[i];
                    reinterpret_cast<float4 *>(sS + SLG * D)[e] = byte16 ? over16(cv[i]) : cv[i];
                }
            }
        }
    }

    const int L_kv = (int)a.L_kv;
    const int nt = (L_kv + AT_NT - 1) / AT_NT;
    // this work-group's KV tiles [t_begin, t_end)
    const int t_begin = a.split_t0[split], t_end = a.split_t0[split + 1];
    const int n_begin = t_begin * AT_NT, g_begin = a.split_g0[split];

    // ---------------- items of 4 tokens: K items plane-fastest, V items
    // token-fastest, which makes both LDS write patterns bank-conflict free.
    // Slot it < NKP is K item it, slot NKP + j is V item j: the kind of an
    // item is the same across a wave.
    const uint32_t *plane[IPT];
    const float *sbase[IPT];
    int it_w[IPT], it_t4[IPT];
    bool it_v[IPT], it_ok[IPT];
#pragma unroll
    for (int r = 0; r < IPT; ++r) {
        const int it = tid + THREADS * r;
        const bool isV = __builtin_amdgcn_readfirstlane(it >= NKP ? 1 : 0) != 0;
        const int j = isV ? it - NKP : it;
        it_ok[r] = j < 16 * W && it < NSLOTS;
        it_v[r] = isV;
        it_w[r] = isV ? (j >> 4) : (j % W);
        it_t4[r] = isV ? (j & 15) : (j / W);
        if (!it_ok[r]) { it_w[r] = 0; it_t4[r] = 0; }      // it_v stays the wave's kind
        if constexpr (DENSE)
            plane[r] = reinterpret_cast<const uint32_t *>((it_v[r] ? a.vd : a.kd) + (int64_t)bh * a.L_cap * D +
                                                          it_w[r] * CPW);
        else
            plane[r] = (it_v[r] ? a.pv : a.pk) + ((int64_t)bh * W + it_w[r]) * a.L_cap;
        sbase[r] = DENSE ? nullptr : (it_v[r] ? a.sv : a.sk) + (int64_t)bh * a.G_cap * D + it_w[r] * CPW;
    }

    // Prefetched tile: words per item and, when the tile lies in one block and
    // scales are not in LDS, that block's scales for the item's channels. A
    // tile's loads are issued right after the tile before it is staged, a
    // whole tile's compute ahead of their use.
    struct Pref {
        uint32_t wd[IPT][T::WORDS];
        float sc[IPT][CPW];
        int g;        // block of the tile's first token
        bool split;   // the tile contains a block boundary
    };
    Pref P0;
    P0.g = 0;
    P0.split = false;
    // block of the last prefetched tile and its end (the next block's first
    // token), kept in registers: only a tile past that end reads the block
    // table again
    int g_run = a.split_g0[split];
    int e_run = a.off[g_run + 1];

    // words of the (packed) tile at n0 whose first token is in block g and,
    // when scales are not in LDS, that block's scales for the item's channels
    auto prefetch_words = [&](Pref &P, int n0, int g, bool split) {
        P.g = g;
        P.split = split;
#pragma unroll
        for (int r = 0; r < IPT; ++r) {
            if (!it_ok[r]) continue;
            const uint4 v0 = *reinterpret_cast<const uint4 *>(plane[r] + attn_item_first_token(n0, it_t4[r], L_kv));
            P.wd[r][0] = v0.x; P.wd[r][1] = v0.y; P.wd[r][2] = v0.z; P.wd[r][3] = v0.w;
            if constexpr (SL) continue;
            const float *srow = sbase[r] + P.g * D;
            if constexpr (D % CPW == 0) {
                // whole words only: the item's scales are one contiguous run
                if constexpr (CPW % 4 == 0) {
#pragma unroll
                    for (int i = 0; i < CPW; i += 4) {
                        const float4 v = *reinterpret_cast<const float4 *>(srow + i);
                        P.sc[r][i] = v.x; P.sc[r][i + 1] = v.y; P.sc[r][i + 2] = v.z; P.sc[r][i + 3] = v.w;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < CPW; ++i) P.sc[r][i] = srow[i];
                }
            } else {
                const int ncw = min(CPW, D - it_w[r] * CPW);
#pragma unroll
                for (int i = 0; i < CPW; ++i) P.sc[r][i] = srow[min(i, ncw - 1)];
            }
        }
    };

    // words of tile n0 (items past the window re-read its last 4-token group,
    // so no load leaves the cache) and, for a tile inside one block, that
    // block's scales
    auto prefetch = [&](Pref &P, int n0) {
        if constexpr (DENSE) {
            // 4 rows of 8 channels per item; rows past L_kv re-read the last
            // row (masked in compute): the dense buffer has exactly L_cap rows
#pragma unroll
            for (int r = 0; r < IPT; ++r) {
                if (!it_ok[r]) continue;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int t = min(n0 + 4 * it_t4[r] + k, L_kv - 1);
                    const uint4 v = *reinterpret_cast<const uint4 *>(plane[r] + (int64_t)t * (D / 2));
                    P.wd[r][4 * k] = v.x; P.wd[r][4 * k + 1] = v.y; P.wd[r][4 * k + 2] = v.z; P.wd[r][4 * k + 3] = v.w;
                }
            }
            return;
        }
        while (e_run <= n0) e_run = off[++g_run + 1];
        prefetch_words(P, n0, g_run, e_run < min(n0 + AT_NT, L_kv));
    };

    // Tile 0's words, the queries and the LDS-bound scales are all in flight
    // before the first wait.
    if constexpr (!DENSE) prefetch_words(P0, n_begin, g_begin, a.off[g_begin + 1] < min(n_begin + AT_NT, L_kv));

    // Q^T operands: lane = query, slots (hf, j) = channel 16*ks + 8*hf + j
    const int q_base = qt * QT + wave * QW + lr;
    // a wave whose queries all lie past Lq (the last query tile of a block
    // that is not a multiple of the tile) only helps dequantize tiles into LDS
    const bool wave_idle = __builtin_amdgcn_readfirstlane(qt * QT + wave * QW) >= a.Lq;
    bf16x8 qop[QB][KSTEPS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qi = q_base + 32 * qb;
        const uint16_t *qrow = a.q + (int64_t)b * a.sq_b + (int64_t)qi * a.sq_l + (int64_t)h * a.sq_h + 8 * hf;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (qi < a.Lq) v = *reinterpret_cast<const uint4 *>(qrow + 16 * ks);
            qop[qb][ks] = as_bf16x8(v);
        }
    }

    // Retire these loads here. Otherwise the wait-count analysis sees them
    // pending at the loop header and waits for every outstanding load (the
    // KV prefetch included) before the first matrix-core op of each tile.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

    if constexpr (SL) {
        if constexpr (SLP == 1) {
            const bool mine = tid < a.G * (D / 4);
            byte16 = BITS == 4 && __syncthreads_and(!mine || (div16_exact(sl_k) && div16_exact(sl_v)) ? 1 : 0) != 0;
            if (mine) {
                reinterpret_cast<float4 *>(sS)[tid] = byte16 ? over16(sl_k) : sl_k;
                reinterpret_cast<float4 *>(sS + SLG * D)[tid] = byte16 ? over16(sl_v) : sl_v;
            }
        }
    }

    floatx16 o[QB][DBLK];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int d = 0; d < DBLK; ++d)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[qb][d][r] = 0.0f;
    float m_run[QB], l_run[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) { m_run[qb] = -INFINITY; l_run[qb] = 0.0f; }

    __syncthreads();   // off[] (and scales in LDS) ready

    // item r of a prefetched tile into LDS buffer `buf`; scale of code i of
    // token k is sk(k, i)
    auto dequant_item = [&](int buf, const Pref &P, int r, auto sk) {
        uint16_t *K = Ks + buf * KBUF;
        uint16_t *V = Vt + buf * VBUF;
        const int w = it_w[r], t4 = it_t4[r];
        const int cbase = w * CPW;
        const int ncw = min(CPW, D - cbase);
        if (it_v[r]) {
            const int p0 = v_pos(4 * t4);
#pragma unroll
            for (int i = 0; i < CPW; ++i) {
                if (i < ncw) {
                    uint2 lo;
                    lo.x = pack_bf16x2(field_f32<BITS>(P.wd[r][0], i) * sk(0, i), field_f32<BITS>(P.wd[r][1], i) * sk(1, i));
                    lo.y = pack_bf16x2(field_f32<BITS>(P.wd[r][2], i) * sk(2, i), field_f32<BITS>(P.wd[r][3], i) * sk(3, i));
                    *reinterpret_cast<uint2 *>(V + (cbase + i) * VP + p0) = lo;
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                uint16_t *dst = K + (4 * t4 + k) * KP + cbase;
                uint32_t pw[(CPW + 1) / 2];
#pragma unroll
                for (int i = 0; i < CPW; i += 2) {
                    const float v0 = field_f32<BITS>(P.wd[r][k], i) * sk(k, i);
                    const float v1 = (i + 1 < CPW) ? field_f32<BITS>(P.wd[r][k], i + 1) * sk(k, i + 1) : 0.0f;
                    pw[i / 2] = pack_bf16x2(v0, v1);
                }
                if constexpr (CPW % 8 == 0) {
#pragma unroll
                    for (int i = 0; i < CPW / 2; i += 4)
                        *reinterpret_cast<uint4 *>(dst + 2 * i) = make_uint4(pw[i], pw[i + 1], pw[i + 2], pw[i + 3]);
                } else if constexpr (CPW % 4 == 0) {
#pragma unroll
                    for (int i = 0; i < CPW / 2; i += 2)
                        *reinterpret_cast<uint2 *>(dst + 2 * i) = make_uint2(pw[i], pw[i + 1]);
                } else if constexpr (CPW % 2 == 0) {
#pragma unroll
                    for (int i = 0; i < CPW / 2; ++i)
                        if (2 * i < ncw) *reinterpret_cast<uint32_t *>(dst + 2 * i) = pw[i];
                } else {
#pragma unroll
                    for (int i = 0; i < CPW; ++i)
                        if (i < ncw) dst[i] = (uint16_t)(pw[i / 2] >> (16 * (i & 1)));
                }
            }
        }
    };

    // item r by byte decode (INT8, or INT4 with s / 16 in the LDS table):
    // the same values as dequant_item
    auto dequant_item_bytes = [&](int buf, const Pref &P, int r, const float (&sc)[CPW]) {
        if constexpr (BITS == 4 || BITS == 8) {
            uint16_t *K = Ks + buf * KBUF;
            uint16_t *V = Vt + buf * VBUF;
            const int cbase = it_w[r] * CPW, t4 = it_t4[r];
            if (it_v[r]) {
                const ByteWord<BITS> b0(P.wd[r][0]), b1(P.wd[r][1]), b2(P.wd[r][2]), b3(P.wd[r][3]);
                const int p0 = v_pos(4 * t4);
                static_for<CPW>([&](auto I) {
                    constexpr int i = decltype(I)::value;
                    const float sv = sc[i];
                    const uint2 lo = make_uint2(pack_bf16x2(b0.template field<i>() * sv, b1.template field<i>() * sv),
                                                pack_bf16x2(b2.template field<i>() * sv, b3.template field<i>() * sv));
                    *reinterpret_cast<uint2 *>(V + (cbase + i) * VP + p0) = lo;
                });
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const ByteWord<BITS> bw(P.wd[r][k]);
                    uint32_t pw[CPW / 2];
                    static_for<CPW / 2>([&](auto J) {
                        constexpr int j = decltype(J)::value;
                        pw[j] = pack_bf16x2(bw.template field<2 * j>() * sc[2 * j], bw.template field<2 * j + 1>() * sc[2 * j + 1]);
                    });
                    uint16_t *dst = K + (4 * t4 + k) * KP + cbase;
                    if constexpr (CPW == 8) *reinterpret_cast<uint4 *>(dst) = make_uint4(pw[0], pw[1], pw[2], pw[3]);
                    else *reinterpret_cast<uint2 *>(dst) = make_uint2(pw[0], pw[1]);
                }
            }
        }
    };

    // CPW scales of one block row from LDS (row = that block's D scales,
    // offset by the item's first channel): 16-byte reads when whole words
    // tile the row, the channel past the row's end clamped otherwise
    auto scale_row = [&](float (&dst)[CPW], const float *row, int ncw) {
        if constexpr (D % CPW == 0 && CPW % 4 == 0) {
#pragma unroll
            for (int i = 0; i < CPW; i += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(row + i);
                dst[i] = v.x; dst[i + 1] = v.y; dst[i + 2] = v.z; dst[i + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < CPW; ++i) dst[i] = row[min(i, ncw - 1)];
        }
    };

    // dequantize a prefetched tile starting at token n0 into LDS buffer `buf`
    auto dequant = [&](int buf, const Pref &P, int n0) {
        if constexpr (DENSE) {
            // bf16 rows as they are: K row-major, V transposed
            uint16_t *K = Ks + buf * KBUF;
            uint16_t *V = Vt + buf * VBUF;
#pragma unroll
            for (int r = 0; r < IPT; ++r) {
                if (!it_ok[r]) continue;
                const int c8 = it_w[r] * 8, t4 = it_t4[r];
                if (!it_v[r]) {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        *reinterpret_cast<uint4 *>(K + (4 * t4 + k) * KP + c8) =
                            make_uint4(P.wd[r][4 * k], P.wd[r][4 * k + 1], P.wd[r][4 * k + 2], P.wd[r][4 * k + 3]);
                } else {
                    const int p0 = v_pos(4 * t4);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        // channel c8 + i of tokens 0..3: half i & 1 of word i / 2 of each row
                        const int sh = 16 * (i & 1);
                        const uint32_t e0 = (P.wd[r][i / 2] >> sh) & 0xFFFFu, e1 = (P.wd[r][4 + i / 2] >> sh) & 0xFFFFu;
                        const uint32_t e2 = (P.wd[r][8 + i / 2] >> sh) & 0xFFFFu, e3 = (P.wd[r][12 + i / 2] >> sh) & 0xFFFFu;
                        *reinterpret_cast<uint2 *>(V + (c8 + i) * VP + p0) = make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
                    }
                }
            }
            return;
        }
#pragma unroll
        for (int r = 0; r < IPT; ++r) {
            if (!it_ok[r]) continue;
            const int cbase = it_w[r] * CPW;
            const int ncw = min(CPW, D - cbase);
            if constexpr (SL) {
                // scale rows in LDS: one per token (the tile's block unless split)
                const float *base = sS + (it_v[r] ? SLG * D : 0) + cbase;
                if (!P.split) {
                    float scl[CPW];
                    scale_row(scl, base + P.g * D, ncw);
                    if constexpr (BITS == 8) {
                        dequant_item_bytes(buf, P, r, scl);
                    } else if constexpr (BITS == 4) {
                        if (byte16) dequant_item_bytes(buf, P, r, scl);
                        else dequant_item(buf, P, r, [&](int, int i) { return scl[i]; });
                    } else {
                        dequant_item(buf, P, r, [&](int, int i) { return scl[i]; });
                    }
                } else {
                    // a tile with a block boundary: each token takes the scale
                    // row of its own block; the same vector path for every item,
                    // so no lane of a wave waits on a slower one
                    const int t0 = n0 + 4 * it_t4[r];
                    int g = P.g;
                    if constexpr (CPW <= 8) {
                        // up to 32 scales: held in registers
                        float scl[4][CPW];
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            g = group_of(off, g, min(t0 + k, L_kv - 1));
                            scale_row(scl[k], base + g * D, ncw);
                        }
                        // a table of s / 16 (exact) gives back s times 16
                        const float tm = byte16 ? 16.0f : 1.0f;
                        dequant_item(buf, P, r, [&](int k, int i) { return scl[k][i] * tm; });
                    } else {
                        // wider words: scales read where used, to bound registers
                        const float *row[4];
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            g = group_of(off, g, min(t0 + k, L_kv - 1));
                            row[k] = base + g * D;
                        }
                        dequant_item(buf, P, r, [&](int k, int i) { return row[k][min(i, ncw - 1)]; });
                    }
                }
            } else if (!P.split) {
                dequant_item(buf, P, r, [&](int, int i) { return P.sc[r][i]; });
            } else {
                // a tile with a block boundary (rare at this head_dim): per-token
                // scale rows from memory, one token at a time to bound registers
                uint16_t *K = Ks + buf * KBUF;
                uint16_t *V = Vt + buf * VBUF;
                const int t4 = it_t4[r];
                int g = P.g;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    g = group_of(off, g, min(n0 + 4 * t4 + k, L_kv - 1));
                    const float *srow = sbase[r] + g * D;
#pragma unroll
                    for (int i = 0; i < CPW; ++i) {
                        if (i < ncw) {
                            const float v = field_f32<BITS>(P.wd[r][k], i) * srow[i];
                            const uint16_t bits16 = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
                            if (it_v[r]) V[(cbase + i) * VP + v_pos(4 * t4 + k)] = bits16;
                            else K[(4 * t4 + k) * KP + cbase + i] = bits16;
                        }
                    }
                }
            }
        }
    };

    const float c = a.scale_log2;
    // one 64-token tile from LDS buffer `buf`. The matrix core and the vector
    // ALUs only overlap when their instructions alternate within one wave, so
    // the tile is issued as: scores of half 0; scores of half 1 interleaved
    // with the exponentials of half 0; P*V of half 0 interleaved with the
    // exponentials of half 1; P*V of half 1.
    auto compute = [&](int buf, int n0, bool masked) __attribute__((always_inline)) {
        if (wave_idle) return;
        const uint16_t *Kb = Ks + buf * KBUF + lr * KP + 8 * hf;
        const uint16_t *Vb = Vt + buf * VBUF + lr * VP + 8 * hf;
        floatx16 s[2][QB];
        bf16x8 pop[2][QB][2];
        float lt[2][QB];
        auto mask = [&](int tb) {
            if (masked) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int tok = n0 + 32 * tb + 8 * (r >> 2) + 4 * hf + (r & 3);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        if (tok >= L_kv) s[tb][qb][r] = -INFINITY;
                }
            }
        };
        // exponentials of half tb against the running maximum, element pairs
        // [j0, j0 + nj) of the flattened (query block, pair) index; packed bf16
        // p go to uu, their sum to lt
        uint32_t uu[2][QB][8];
        auto exps_part = [&](int tb, int j0, int nj) {
#pragma unroll
            for (int j = j0; j < j0 + nj; ++j) {
                const int qb = j / 8, e = j % 8;
                const float mneg = -m_run[qb];
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[tb][qb][2 * e], c, mneg));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[tb][qb][2 * e + 1], c, mneg));
                uu[tb][qb][e] = pack_bf16x2(p0, p1);
                lt[tb][qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, uu[tb][qb][e]), ones_bf16x2(),
                                                             lt[tb][qb], false);
            }
        };
        auto exps = [&](int tb, int qb) {
            lt[tb][qb] = 0.0f;
            exps_part(tb, 8 * qb, 8);
        };
        auto make_pop = [&](int tb) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    pop[tb][qb][hh] = as_bf16x8(make_uint4(uu[tb][qb][4 * hh], uu[tb][qb][4 * hh + 1],
                                                           uu[tb][qb][4 * hh + 2], uu[tb][qb][4 * hh + 3]));
        };
        // The running maximum is raised only when a half's exponentials leave
        // [0, 2^64): on the first tile (m_run = -inf gives inf or NaN) or when
        // scores grow by more than 64 in log2 units. Below that bound p, l and
        // o stay far from fp32 overflow, and fp32/bf16 relative precision does
        // not depend on the offset, so no per-tile maximum is needed.
        auto settle = [&](int tb) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                if (__builtin_amdgcn_ballot_w64(!(lt[tb][qb] < 0x1p64f)) != 0) {
                    // scores are finite or -inf (masked), never NaN
                    float mx = __builtin_elementwise_maximum(s[tb][qb][0], s[tb][qb][1]);
#pragma unroll
                    for (int r = 2; r < 16; r += 2)
                        mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(s[tb][qb][r], s[tb][qb][r + 1]));
                    const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, mx),
                                                                     __builtin_bit_cast(uint32_t, mx), false, false);
                    mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(__builtin_bit_cast(float, (uint32_t)sw[0]),
                                                                                         __builtin_bit_cast(float, (uint32_t)sw[1])));
                    const float m_new = fmaxf(m_run[qb], mx * c);
                    const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
                    m_run[qb] = m_new;
                    l_run[qb] *= alpha;
#pragma unroll
                    for (int d = 0; d < DBLK; ++d) scale_acc16(o[qb][d], alpha);
                    exps(tb, qb);
                }
                l_run[qb] += lt[tb][qb];
            }
            make_pop(tb);
        };
        auto kread = [&](int tb, int ks) {
            return as_bf16x8(*reinterpret_cast<const uint4 *>(Kb + 32 * tb * KP + 16 * ks));
        };
        auto vread = [&](int tb, int i) {     // i = 2 * d + hh
            return as_bf16x8(*reinterpret_cast<const uint4 *>(Vb + 32 * (i >> 1) * VP + 32 * tb + 16 * (i & 1)));
        };
        auto pv = [&](int tb) {
#pragma unroll
            for (int i = 0; i < 2 * DBLK; ++i) {
                const bf16x8 va = vread(tb, i);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    o[qb][i >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pop[tb][qb][i & 1], o[qb][i >> 1], 0, 0, 0);
            }
        };

        // half 0: scores, LDS operands read AT_RA steps ahead
        {
            bf16x8 kop[AT_RA + 1];
#pragma unroll
            for (int i = 0; i < AT_RA && i < KSTEPS; ++i) kop[i] = kread(0, i);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < KSTEPS; ++k) {
                if (k + AT_RA < KSTEPS) kop[(k + AT_RA) % (AT_RA + 1)] = kread(0, k + AT_RA);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    s[0][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[k % (AT_RA + 1)], qop[qb][k],
                                                                       k == 0 ? floatx16{} : s[0][qb], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        mask(0);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) { lt[0][qb] = 0.0f; lt[1][qb] = 0.0f; s[1][qb] = floatx16{}; }
        // half 1 scores on the matrix core || half 0 exponentials on the VALU;
        // the LDS operand of step k + 1 is read during step k
        {
            constexpr int NS = KSTEPS;                  // matrix steps (x QB ops each)
            constexpr int NJ = 8 * QB;                  // exponential pairs
            bf16x8 kop[AT_RA + 1];
#pragma unroll
            for (int i = 0; i < AT_RA && i < NS; ++i) kop[i] = kread(1, i);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                if (k + AT_RA < NS) kop[(k + AT_RA) % (AT_RA + 1)] = kread(1, k + AT_RA);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    s[1][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[k % (AT_RA + 1)], qop[qb][k], s[1][qb], 0, 0, 0);
                exps_part(0, NJ * k / NS, NJ * (k + 1) / NS - NJ * k / NS);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        settle(0);
        mask(1);
        // half 0 P*V on the matrix core || half 1 exponentials on the VALU
        {
            constexpr int NS = 2 * DBLK;
            constexpr int NJ = 8 * QB;
            bf16x8 vop[AT_RA + 1];
#pragma unroll
            for (int i = 0; i < AT_RA && i < NS; ++i) vop[i] = vread(0, i);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < NS; ++k) {
                if (k + AT_RA < NS) vop[(k + AT_RA) % (AT_RA + 1)] = vread(0, k + AT_RA);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    o[qb][k >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[k % (AT_RA + 1)], pop[0][qb][k & 1], o[qb][k >> 1], 0, 0, 0);
                exps_part(1, NJ * k / NS, NJ * (k + 1) / NS - NJ * k / NS);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        settle(1);
        pv(1);
    };

    // pre-RoPE: rotate the K pairs of the tile in LDS buffer `buf` (tokens past
    // L_kv take the last row's angles; the scores mask them)
    auto rope_tile = [&](int buf, int n0) {
        uint16_t *K = Ks + buf * KBUF;
        constexpr int HALF = D / 2, PAIRS = AT_NT * HALF;
#pragma unroll
        for (int p0 = 0; p0 < PAIRS; p0 += THREADS) {
            const int p = p0 + tid;
            const int tok = p / HALF, i = p - tok * HALF;
            const int64_t trow = (int64_t)min(n0 + tok, L_kv - 1) * HALF + i;
            const float c = a.rcos[trow], s = a.rsin[trow];
            uint32_t *kp = reinterpret_cast<uint32_t *>(K + tok * KP + 2 * i);
            const uint32_t v = *kp;
            const float x0 = bf16lo(v), x1 = bf16hi(v);
            const float c0 = x0 * c, c1 = x1 * s, c2 = x0 * s, c3 = x1 * c;
            *kp = pack_bf16x2(c0 - c1, c2 + c3);
        }
    };

    // ---------------- pipeline: LDS-only barrier (global prefetches stay in
    // flight); tile jt + 2 is prefetched while tile jt is computed and tile
    // jt + 1 dequantized into the other LDS buffer. With ROPE, a tile is
    // rotated in place (one more barrier) before its compute.
    auto lds_barrier = []() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
    int jt = t_begin;
    if constexpr (DENSE) prefetch(P0, n_begin);
    dequant(0, P0, n_begin);
    if (t_begin + 1 < t_end) prefetch(P0, n_begin + AT_NT);
    lds_barrier();
    for (; jt + 1 < t_end; ++jt) {
        const int cur = (jt - t_begin) & 1;
        const int n0 = jt * AT_NT;
        if constexpr (ROPE) {
            rope_tile(cur, n0);
            lds_barrier();
        }
        // the next tile's staging follows this tile's compute and overlaps
        // its last matrix ops (dequantization interleaved with the matrix ops
        // of the exponential-free phases measured slower)
        compute(cur, n0, false);
        dequant(cur ^ 1, P0, n0 + AT_NT);
        if (jt + 2 < t_end) prefetch(P0, n0 + 2 * AT_NT);
        lds_barrier();
    }
    if constexpr (ROPE) {
        rope_tile((jt - t_begin) & 1, jt * AT_NT);
        lds_barrier();
    }
    compute((jt - t_begin) & 1, jt * AT_NT, jt + 1 == nt);

    // ---------------- one KV range of several: unnormalized O and (m, l)
    if (a.kv_splits > 1) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int qi = q_base + 32 * qb;
            const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
            if (qi < a.Lq) {
                const int64_t row = ((int64_t)split * a.B * a.H + bh) * a.Lq + qi;
                float *po = a.part_o + row * D;
#pragma unroll
                for (int d = 0; d < DBLK; ++d) {
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) {
                        const int ch = 32 * d + 8 * r4 + 4 * hf;
                        *reinterpret_cast<float4 *>(po + ch) =
                            make_float4(o[qb][d][4 * r4], o[qb][d][4 * r4 + 1], o[qb][d][4 * r4 + 2], o[qb][d][4 * r4 + 3]);
                    }
                }
                if (hf == 0) *reinterpret_cast<float2 *>(a.part_ml + 2 * row) = make_float2(m_run[qb], l_tot);
            }
        }
        return;
    }

    // ---------------- normalise and store
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qi = q_base + 32 * qb;
        const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
        const float inv = 1.0f / l_tot;
        if (qi < a.Lq) {
            uint16_t *orow = a.out + (int64_t)b * a.so_b + (int64_t)qi * a.so_l + (int64_t)h * a.so_h;
#pragma unroll
            for (int d = 0; d < DBLK; ++d) {
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int ch = 32 * d + 8 * r4 + 4 * hf;
                    uint2 v;
                    v.x = pack_bf16x2(o[qb][d][4 * r4] * inv, o[qb][d][4 * r4 + 1] * inv);
                    v.y = pack_bf16x2(o[qb][d][4 * r4 + 2] * inv, o[qb][d][4 * r4 + 3] * inv);
                    *reinterpret_cast<uint2 *>(orow + ch) = v;
                }
            }
        }
    }
}

// Combine the KV ranges of a split launch: with m* the largest range maximum
// and w_s = 2^(m_s - m*), O = sum_s w_s O_s / sum_s w_s l_s, stored as bf16.
// One thread per 4 channels of one (batch, head, query).
__global__ __launch_bounds__(256) void merge_kv_splits(const AttnArgs a, int D) {
    const int64_t q4 = D / 4;
    const int64_t n = (int64_t)a.B * a.H * a.Lq * q4;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int c4 = (int)(i % q4);
    const int64_t bhq = i / q4;                        // (b*H + h) * Lq + qi
    const int qi = (int)(bhq % a.Lq);
    const int bh = (int)(bhq / a.Lq);
    const int b = bh / a.H, h = bh % a.H;
    const int64_t stride = (int64_t)a.B * a.H * a.Lq;  // rows per split
    float m_star = -INFINITY;
    for (int s = 0; s < a.kv_splits; ++s) m_star = fmaxf(m_star, a.part_ml[2 * (s * stride + bhq)]);
    float l = 0.0f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < a.kv_splits; ++s) {
        const int64_t row = s * stride + bhq;
        const float2 ml = *reinterpret_cast<const float2 *>(a.part_ml + 2 * row);
        const float w = __builtin_amdgcn_exp2f(ml.x - m_star);
        const float4 v = *reinterpret_cast<const float4 *>(a.part_o + row * D + 4 * c4);
        l = __builtin_fmaf(w, ml.y, l);
        acc.x = __builtin_fmaf(w, v.x, acc.x); acc.y = __builtin_fmaf(w, v.y, acc.y);
        acc.z = __builtin_fmaf(w, v.z, acc.z); acc.w = __builtin_fmaf(w, v.w, acc.w);
    }
    const float inv = 1.0f / l;
    uint16_t *orow = a.out + (int64_t)b * a.so_b + (int64_t)qi * a.so_l + (int64_t)h * a.so_h + 4 * c4;
    uint2 v;
    v.x = pack_bf16x2(acc.x * inv, acc.y * inv);
    v.y = pack_bf16x2(acc.z * inv, acc.w * inv);
    *reinterpret_cast<uint2 *>(orow) = v;
}

#ifndef VARQ_ATTN_QB
#define VARQ_ATTN_QB 1
#endif
#ifndef VARQ_ATTN_NW
#define VARQ_ATTN_NW 8
#endif
constexpr int AT_CFG_QB = VARQ_ATTN_QB;
constexpr int AT_CFG_NW = VARQ_ATTN_NW;

template <int BITS, int D>
static hipError_t launch_at(const AttnArgs &a, hipStream_t st) {
    const int64_t n_blocks = (int64_t)a.n_qtiles * a.B * a.H * a.kv_splits;
    const int64_t grid = (n_blocks + 7) / 8 * 8;
    if (a.rcos) {
        hipLaunchKernelGGL((packed_attention_v5<BITS, D, AT_CFG_QB, AT_CFG_NW, false, true>), dim3((unsigned)grid),
                           dim3(64 * AT_CFG_NW), 0, st, a);
        return hipGetLastError();
    }
    // up to at_sl_maxg<D>() blocks' scales live in LDS; otherwise scales
    // stream with the words
    if (a.G <= at_sl_maxg<D>())
        hipLaunchKernelGGL((packed_attention_v5<BITS, D, AT_CFG_QB, AT_CFG_NW, true>), dim3((unsigned)grid),
                           dim3(64 * AT_CFG_NW), 0, st, a);
    else
        hipLaunchKernelGGL((packed_attention_v5<BITS, D, AT_CFG_QB, AT_CFG_NW, false>), dim3((unsigned)grid),
                           dim3(64 * AT_CFG_NW), 0, st, a);
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

int attention_q_tile() { return 32 * AT_CFG_QB * AT_CFG_NW; }

// Dense bf16 K/V (the unfused baseline): the same pipeline and compute, with
// tiles staged from bf16 rows instead of dequantized from packed words.
hipError_t launch_dense_attention(const AttnArgs &a, int D, hipStream_t st) {
    const int64_t n_blocks = (int64_t)a.n_qtiles * a.B * a.H * a.kv_splits;
    const int64_t grid = (n_blocks + 7) / 8 * 8;
    if (D == 64)
        hipLaunchKernelGGL((packed_attention_v5<16, 64, AT_CFG_QB, AT_CFG_NW, false>), dim3((unsigned)grid),
                           dim3(64 * AT_CFG_NW), 0, st, a);
    else if (D == 128)
        hipLaunchKernelGGL((packed_attention_v5<16, 128, AT_CFG_QB, AT_CFG_NW, false>), dim3((unsigned)grid),
                           dim3(64 * AT_CFG_NW), 0, st, a);
    else
        return hipErrorInvalidValue;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.kv_splits == 1) return e;
    const int64_t n = (int64_t)a.B * a.H * a.Lq * (D / 4);
    hipLaunchKernelGGL(merge_kv_splits, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a, D);
    return hipGetLastError();
}

hipError_t launch_packed_attention(const AttnArgs &a, int D, int bits, hipStream_t st) {
    hipError_t e = hipErrorInvalidValue;
    if (D == 64) e = launch_at_bits<64>(a, bits, st);
    if (D == 128) e = launch_at_bits<128>(a, bits, st);
    if (e != hipSuccess || a.kv_splits == 1) return e;
    const int64_t n = (int64_t)a.B * a.H * a.Lq * (D / 4);
    hipLaunchKernelGGL(merge_kv_splits, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a, D);
    return hipGetLastError();
}

}  // namespace varq
