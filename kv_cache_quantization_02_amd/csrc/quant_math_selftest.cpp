// quant_math_selftest.cpp - host-only exhaustive check of the scalar arithmetic
// the gfx950 kernels use for codes (varq_quant_math.h), and of the attention's
// tile-load indices (varq_tile_math.h).
//
// For every positive finite bf16 absmax a and every bf16 x with |x| <= a, the
// kernels' code for x under s = fp32(a / qmax) must equal rint(fl32(x / s))
// computed with the host's IEEE division. Negative x follow by symmetry of both
// rounding steps. Scales below kFastScaleMin take the division path in the
// kernels and are checked through code_exact(). The bit-pattern forms that the
// packers use must carry the same code in their low 8 bits, for x and -x.
#include <stdint.h>

#include <atomic>
#include <cmath>
#include <thread>
#include <vector>

#include "varq_quant_math.h"
#include "varq_tile_math.h"

namespace {

inline float bf16_to_f32(uint32_t b) { return varq::u2f(b << 16); }

}  // namespace

extern "C" {

// Returns the number of (x, a) pairs whose kernel code differs from the IEEE
// reference for this bit width (0 expected); *checked receives the pair count.
long long varq_selftest_codes_exhaustive(int bits, int n_threads, long long *checked) {
    if (bits < 2 || bits > 8) return -1;
    const float qm = (float)((1 << (bits - 1)) - 1);
    if (n_threads < 1) n_threads = 1;
    std::atomic<long long> bad{0}, total{0};
    auto work = [&](int tid) {
        long long lb = 0, lt = 0;
        for (uint32_t a16 = 1 + tid; a16 < 0x7F80u; a16 += n_threads) {
            const float a = bf16_to_f32(a16);
            const float s = a / qm;
            const float y = varq::recip_for_codes(s);
            const bool fast = varq::fast_scale_ok(s);
            for (uint32_t x16 = 0; x16 <= a16; ++x16) {
                const float x = bf16_to_f32(x16);
                const int32_t got = fast ? varq::code_fast(x, s, y) : varq::code_exact(x, s);
                const int32_t ref = (int32_t)std::nearbyint(x / s);
                // the packers keep the low bits of the rounded float's pattern:
                // they must be the code's two's complement low bits, for x and -x
                const uint32_t gp = fast ? varq::code_fast_bits(x, s, y) : varq::code_exact_bits(x, s);
                const uint32_t gn = fast ? varq::code_fast_bits(-x, s, y) : varq::code_exact_bits(-x, s);
                lb += (got != ref) || ((gp ^ (uint32_t)ref) & 0xFFu) != 0 || ((gn ^ (uint32_t)-ref) & 0xFFu) != 0;
                ++lt;
            }
        }
        bad += lb;
        total += lt;
    };
    std::vector<std::thread> th;
    for (int t = 0; t < n_threads; ++t) th.emplace_back(work, t);
    for (auto &t : th) t.join();
    if (checked) *checked = total.load();
    return bad.load();
}

// Dequantization: bf16 pattern of fl32(q * s) for every code of the bit width
// and fp32 scales spread over the patterns [lo16, hi16) of their high halves,
// compared with the nearest of the product's two bf16 neighbours (ties to the
// even pattern). Products beyond the largest finite bf16 cannot occur.
long long varq_selftest_dequant(int bits, uint32_t lo16, uint32_t hi16) {
    if (bits < 2 || bits > 8) return -1;
    const int qm = (1 << (bits - 1)) - 1;
    long long bad = 0;
    for (uint32_t s16 = lo16; s16 < hi16; ++s16) {
        for (uint32_t lowbits = 0; lowbits < 0x10000u; lowbits += 0x1111u) {
            const float s = varq::u2f((s16 << 16) | lowbits);   // fp32 scales, not only bf16 ones
            for (int q = -qm; q <= qm; ++q) {
                const float p = (float)q * s;
                // |q * s| never exceeds the group's absmax, a finite bf16 value
                if (!(std::fabs(p) <= 3.38953139e38f)) continue;
                const uint32_t got = varq::dequant_bits(q, s);
                // reference: nearest bf16 by comparing the two neighbours in double
                const uint32_t u = varq::f2u(p);
                const uint32_t lo = u & 0xFFFF0000u, hi = lo + 0x10000u;
                const double dl = std::fabs((double)p - (double)varq::u2f(lo));
                const double dh = std::fabs((double)p - (double)varq::u2f(hi));
                uint32_t ref = (dl < dh) ? lo : (dh < dl) ? hi : (((lo >> 16) & 1u) ? hi : lo);
                bad += (got != (ref >> 16));
            }
        }
    }
    return bad;
}

// Highest cache token that the packed attention's tile loads read for a window
// of L_kv tokens (every tile of the window, every item of a tile), with the
// kernel's own index function. Must stay below the cache capacity.
long long varq_selftest_attn_max_token(int L_kv) {
    if (L_kv < 1) return -1;
    const int nt = (L_kv + varq::kAttnTileTokens - 1) / varq::kAttnTileTokens;
    long long hi = -1;
    for (int jt = 0; jt < nt; ++jt)
        for (int t4 = 0; t4 < varq::kAttnTileTokens / varq::kAttnItemTokens; ++t4) {
            const int t = varq::attn_item_first_token(jt * varq::kAttnTileTokens, t4, L_kv);
            if (t % varq::kAttnItemTokens) return -2;          // 16-byte alignment lost
            const long long last = (long long)t + varq::kAttnItemTokens - 1;
            if (last > hi) hi = last;
        }
    return hi;
}

}  // extern "C"
