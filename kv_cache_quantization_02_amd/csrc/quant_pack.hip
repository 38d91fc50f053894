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
// quotient and writes whole words: at 4, 7 and 8 bits a lane's 8 channels
// form whole words directly; at 2, 3, 5 and 6 bits the fields are staged in
// LDS as code bytes and assembled into words. Either way the lanes
// of a work-group cover every token of the unit in each word plane. When every
// block fits one unit, a second tensor of the same shape and block map (V next
// to K) can ride in the same launch: unit ids past the first tensor's units
// address the second tensor's input, words and scales.
//
// A block split over several chunks needs the maximum over all of them. Each
// chunk publishes its partial maxima in a scratch slot tagged with this
// launch's epoch. The work-group holding the block's last chunk then gathers
// the partials with all its threads (waiting on each tag, merging in LDS),
// publishes the block maximum the same way and quantizes its rows; the
// work-group of every other chunk waits for that maximum and quantizes its
// rows. A work-group holds only its current unit, as for whole blocks. Each
// value crosses work-groups in one 64-bit atomic word carrying both the tag
// and the maximum, so no cache flush or fence is needed for it; the epoch
// advances once per launch, set by the last work-group to finish.
//
// Progress (such launches are cooperative: every work-group is resident, and
// no block has more chunks than there are work-groups, G). Work-group w takes
// units w, w + G, ... (round k = units kG .. kG + G - 1); a block's chunks are
// consecutive units, so it lies in one round or two adjacent ones. Every unit
// publishes its partial before it waits for anything. A last chunk waits only
// for partials of lower units; another chunk waits for the maximum of its
// block's last chunk, which can lie in the next round only for the one block
// that crosses into it. Suppose every work-group ends rounds < k. Then all
// start round k and publish; gathers in round k end; so do the chunks of
// blocks whose last chunk lies in round k or earlier. Let block A cross into
// round k + 1, r its last chunk. The unit that r's work-group (and that of
// every other chunk of A in round k + 1) takes in round k lies below A's
// first chunk, since A has at most G chunks, in a block ending by round k:
// those work-groups end round k, publish their chunks of A, r's gather ends
// and A's chunks in round k end too. So every work-group ends round k. Spins
// are nevertheless bounded and report a timeout through a status word.
#include <algorithm>
#include <mutex>

#include "varq_device.h"

namespace varq {

constexpr int QP_THREADS = 256;
constexpr int QP_ITEMS = 8;                                  // 16-byte row chunks held per thread
constexpr int QP_UNIT_ELEMS = QP_THREADS * QP_ITEMS * 8;     // 16384 elements per unit
constexpr int QP_MAX_PACK = 8;                               // blocks per packed unit
constexpr int QP_SLOT_R = QP_MAX_PACK;                       // scale slot of a last chunk
constexpr int QP_SLOT_W = QP_MAX_PACK + 1;                   // scale slot of a waiting chunk
constexpr unsigned QP_SPIN_LIMIT = 1u << 22;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Wave-uniform description of a unit.
struct Unit {
    int64_t id, bh;      // id over the launch (both tensors), (batch*H + head)
    int t;               // tensor: 0 = x, 1 = x2 (one launch for K and V)
    int g0, nb;          // first block, number of blocks (> 1 only for packs)
    int c, nc;           // chunk index and chunk count of block g0 (nc == 1 for packs)
    int row0, n;         // first row relative to x, rows
};

// Packs: unit row where local block j + 1 starts (wave-uniform; past nb - 1
// the entries never match).
struct Bounds {
    int b[QP_MAX_PACK - 1];
};

// Block offsets and unit starts live in LDS (copied once per work-group): a
// lookup in the kernel-argument segment is a dependent scalar load that can
// miss to memory at every step of a search. Values read are the same in all
// lanes and are made wave-uniform.
struct Tables {
    const int32_t *off;   // [G + 1] block offsets relative to x
    const int32_t *us;    // [G + 1] unit_start
};

__device__ inline int lds_uniform(const int32_t *p) { return __builtin_amdgcn_readfirstlane(*p); }

__device__ inline Unit unit_of(const QuantPackArgs &a, const Tables &tb, int64_t id) {
    Unit U;
    U.id = id;
    U.t = id >= a.n_units_one;
    if (U.t) id -= a.n_units_one;
    U.bh = id / a.units_per_bh;
    const int r_in = (int)(id - U.bh * a.units_per_bh);
    int lo = 0, hi = a.G;                 // last g with unit_start[g] <= r_in
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (lds_uniform(tb.us + mid) <= r_in) lo = mid; else hi = mid;
    }
    const int T = a.chunk_rows;
    const int o_lo = lds_uniform(tb.off + lo), o_hi = lds_uniform(tb.off + lo + 1);
    if (o_hi - o_lo > T) {
        U.g0 = lo; U.nb = 1;
        U.c = r_in - lds_uniform(tb.us + lo);
        U.nc = (o_hi - o_lo + T - 1) / T;
        U.row0 = o_lo + U.c * T;
        U.n = min(T, o_hi - U.row0);
    } else {
        int g0 = lo;
        while (g0 > 0 && lds_uniform(tb.us + g0 - 1) == r_in) --g0;
        U.g0 = g0; U.nb = lo - g0 + 1;
        U.c = 0; U.nc = 1;
        U.row0 = lds_uniform(tb.off + g0);
        U.n = o_hi - U.row0;
    }
    return U;
}

__device__ inline Bounds bounds_of(const Tables &tb, const Unit &U) {
    Bounds B;
#pragma unroll
    for (int j = 0; j < QP_MAX_PACK - 1; ++j)
        B.b[j] = j + 1 < U.nb ? lds_uniform(tb.off + U.g0 + 1 + j) - U.row0 : 0x7FFFFFFF;
    return B;
}

// Local block (0 .. nb-1) of unit row r.
__device__ inline int local_block(const Bounds &B, int r) {
    int lb = 0;
#pragma unroll
    for (int j = 0; j < QP_MAX_PACK - 1; ++j) lb += r >= B.b[j] ? 1 : 0;
    return lb;
}

// Blocks of a thread's QP_ITEMS consecutive rows r0 .. r0 + QP_ITEMS - 1:
// the block of r0 and a mask with bit k set where row r0 + k starts a block
// (block starts are distinct, so the block of row r0 + k is lb0 plus the set
// bits 1 .. k). Rows past the unit's end stay in its last block.
struct RowBlocks {
    int lb0;
    uint32_t starts;
};

__device__ inline RowBlocks row_blocks(const Bounds &B, int r0) {
    RowBlocks R;
    R.lb0 = local_block(B, r0);
    R.starts = 0;
#pragma unroll
    for (int j = 0; j < QP_MAX_PACK - 1; ++j) {
        const int d = B.b[j] - r0;
        if (d > 0 && d < QP_ITEMS) R.starts |= 1u << d;
    }
    return R;
}

// Work-group barrier that orders LDS only. __syncthreads() also waits for
// every outstanding global memory operation (vmcnt), e.g. the previous
// unit's word stores at each barrier; no wave here reads global memory another
// wave of its work-group wrote, so LDS ordering is all that is needed.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Thread (chunk, rr) holds channels [8 chunk, 8 chunk + 8) of the unit's rows
// [8 rr, 8 rr + 8): consecutive rows, so a thread's rows rarely span two
// blocks of a pack.
struct Lane {
    Tables tb;
    int D;              // head_dim = LDS slot stride
    int chunk, rr, RP, lpr;
    uint32_t xoff;      // byte offset of this lane's 16 bytes within a row
    bool active;
};

// Issue the 16-byte row-chunk loads of unit U into v (all in flight at once).
// Loads are unconditional so that none waits for the one before it: rows past
// the unit's end (and idle lanes) re-read its last row, which changes no
// maximum and is never stored. Addresses are a wave-uniform base plus a 32-bit
// lane offset (the host checks that a unit's rows span < 2^31 bytes).
__device__ inline void load_unit(const QuantPackArgs &a, const Unit &U, uint4 (&v)[QP_ITEMS], const Lane &L) {
    const int64_t b = U.bh / a.H, h = U.bh - b * a.H;
    const uint16_t *x = U.t ? a.x2 : a.x;
    const int64_t sb = U.t ? a.sx2_b : a.sx_b, sl = U.t ? a.sx2_l : a.sx_l, sh = U.t ? a.sx2_h : a.sx_h;
    const char *ubase = reinterpret_cast<const char *>(x + b * sb + h * sh + (int64_t)U.row0 * sl);
    const uint32_t row_bytes = (uint32_t)sl * 2u;
#pragma unroll
    for (int k = 0; k < QP_ITEMS; ++k) {
        const int r = min(L.rr * QP_ITEMS + k, U.n - 1);
        v[k] = *reinterpret_cast<const uint4 *>(ubase + (uint32_t)r * row_bytes + L.xoff);
    }
}

// Word plane p, unit row r of unit U: wave-uniform base plus a 32-bit lane
// offset (the host checks that W * L_cap words span < 2^31 bytes).
__device__ inline uint32_t *word_at(const QuantPackArgs &a, const Unit &U, int p, int r) {
    char *base = reinterpret_cast<char *>((U.t ? a.packed2 : a.packed) + U.bh * a.W * a.L_cap + a.tok_start + U.row0);
    return reinterpret_cast<uint32_t *>(base + (uint32_t)(p * (uint32_t)a.L_cap + r) * 4u);
}

__device__ inline void flush_max(uint32_t *sh_max, int lb, const Lane &L, const u16x2 (&m)[4]) {
    uint32_t *dst = sh_max + lb * L.D + 8 * L.chunk;
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
__device__ inline void unit_absmax(const QuantPackArgs &a, const Unit &U, const Bounds &B, const uint4 (&v)[QP_ITEMS],
                                   const Lane &L, uint32_t *sh_max) {
    if (!L.active) return;
    u16x2 m[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = u16x2{0, 0};
    if (U.nb == 1) {
#pragma unroll
        for (int k = 0; k < QP_ITEMS; ++k) absmax_item(m, v[k]);      // rows past n repeat row n-1
        flush_max(sh_max, 0, L, m);
        return;
    }
    // rows past n repeat row n-1, which lies in the last block
    const RowBlocks R = row_blocks(B, L.rr * QP_ITEMS);
    int cur = R.lb0;
#pragma unroll
    for (int k = 0; k < QP_ITEMS; ++k) {
        if (k > 0 && ((R.starts >> k) & 1u)) {
            flush_max(sh_max, cur, L, m);
#pragma unroll
            for (int j = 0; j < 4; ++j) m[j] = u16x2{0, 0};
            ++cur;
        }
        absmax_item(m, v[k]);
    }
    flush_max(sh_max, cur, L, m);
}

// b-bit two's complement fields (low bits of each word, higher bits garbage)
// of the 8 channels in w under scales s8 and reciprocals y8. FAST_ONLY: the
// division-free quotient is exact for every scale here (the common case);
// otherwise each channel picks it or IEEE division by its scale.
template <bool FAST_ONLY>
__device__ inline void codes8(const uint4 &w, const float (&s8)[8], const float (&y8)[8], uint32_t (&f)[8]) {
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float xl = bf16lo(wv[j]), xh = bf16hi(wv[j]);
        if (FAST_ONLY) {
            f[2 * j] = code_fast_bits(xl, s8[2 * j], y8[2 * j]);
            f[2 * j + 1] = code_fast_bits(xh, s8[2 * j + 1], y8[2 * j + 1]);
        } else {
            f[2 * j] = fast_scale_ok(s8[2 * j]) ? code_fast_bits(xl, s8[2 * j], y8[2 * j])
                                                : code_exact_bits(xl, s8[2 * j]);
            f[2 * j + 1] = fast_scale_ok(s8[2 * j + 1]) ? code_fast_bits(xh, s8[2 * j + 1], y8[2 * j + 1])
                                                        : code_exact_bits(xh, s8[2 * j + 1]);
        }
    }
}

__device__ inline bool load_sy(const float *sh_s, const float *sh_y, int slot, const Lane &L, float (&s8)[8],
                               float (&y8)[8]) {
    const float4 *ps = reinterpret_cast<const float4 *>(sh_s + slot * L.D + 8 * L.chunk);
    const float4 *py = reinterpret_cast<const float4 *>(sh_y + slot * L.D + 8 * L.chunk);
    const float4 s0 = ps[0], s1 = ps[1], y0 = py[0], y1 = py[1];
    s8[0] = s0.x; s8[1] = s0.y; s8[2] = s0.z; s8[3] = s0.w;
    s8[4] = s1.x; s8[5] = s1.y; s8[6] = s1.z; s8[7] = s1.w;
    y8[0] = y0.x; y8[1] = y0.y; y8[2] = y0.z; y8[3] = y0.w;
    y8[4] = y1.x; y8[5] = y1.y; y8[6] = y1.z; y8[7] = y1.w;
    bool fast = true;
#pragma unroll
    for (int j = 0; j < 8; ++j) fast = fast && fast_scale_ok(s8[j]);
    return fast;
}

// Fields of item k of unit U. SIMPLE: one block whose scales all allow the
// division-free quotient, scales already in s8/y8. Otherwise the item's block
// is looked up (packs), and unless the scales of every lane of the wave allow
// the division-free quotient, each channel picks its quotient.
template <bool SIMPLE>
__device__ inline void item_codes(const QuantPackArgs &a, const Unit &U, const Bounds &B, const uint4 &w,
                                  const Lane &L, int r, int slot, const float *sh_s, const float *sh_y,
                                  float (&s8)[8], float (&y8)[8], int &cur, bool &fast, uint32_t (&f)[8]) {
    if (SIMPLE) {
        codes8<true>(w, s8, y8, f);
    } else {
        const int lb = U.nb > 1 ? local_block(B, r) : slot;
        if (lb != cur) { fast = load_sy(sh_s, sh_y, lb, L, s8, y8); cur = lb; }
        if (__all(fast)) codes8<true>(w, s8, y8, f);
        else codes8<false>(w, s8, y8, f);
    }
}

// Words of unit U formed in registers, written to LDS as sh_w[plane * wp + row].
// MODE: QM_SIMPLE one block, scales in s8/y8, every scale allows the
// division-free quotient; QM_PACK several blocks, every scale of the unit
// allows it (scales reloaded where a thread's rows enter the next block);
// QM_GENERIC anything else (per-row block lookup and per-channel choice).
enum { QM_SIMPLE = 0, QM_PACK = 1, QM_GENERIC = 2 };

template <int BITS, int MODE>
__device__ inline void stage_words(const QuantPackArgs &a, const Unit &U, const Bounds &B, const uint4 (&v)[QP_ITEMS],
                                   const Lane &L, int slot, const float *sh_s, const float *sh_y,
                                   float (&s8)[8], float (&y8)[8], int cur, bool fast, uint32_t *sh_w, int wp) {
    RowBlocks R = {0, 0u};
    if constexpr (MODE == QM_PACK) {
        R = row_blocks(B, L.rr * QP_ITEMS);
        cur = R.lb0;
        if (L.active) load_sy(sh_s, sh_y, cur, L, s8, y8);
    }
#pragma unroll
    for (int k = 0; k < QP_ITEMS; ++k) {
        const int r = L.rr * QP_ITEMS + k;
        const bool live = L.active && r < U.n;
        uint32_t f[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = 0;
        if constexpr (MODE == QM_SIMPLE) {
            // rows past n repeat row n-1; their fields are discarded below
            item_codes<true>(a, U, B, v[k], L, r, slot, sh_s, sh_y, s8, y8, cur, fast, f);
        } else if constexpr (MODE == QM_PACK) {
            if (k > 0 && ((R.starts >> k) & 1u)) {
                ++cur;
                if (L.active) load_sy(sh_s, sh_y, cur, L, s8, y8);
            }
            codes8<true>(v[k], s8, y8, f);
        } else if (live) {
            item_codes<false>(a, U, B, v[k], L, r, slot, sh_s, sh_y, s8, y8, cur, fast, f);
        }
        // Fields enter a word from the top: alignbit(f, w, BITS) = (w >> BITS) |
        // (f << (32 - BITS)) keeps exactly the low BITS bits of f, so after the
        // last field, field j sits at bit BITS * j plus whatever room is left
        // below (32 - BITS * fields); one instruction per field.
        if constexpr (BITS == 4) {
            uint32_t w = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) w = __builtin_amdgcn_alignbit(f[j], w, 4);
            if (live) sh_w[L.chunk * wp + r] = w;
        } else if constexpr (BITS == 7 || BITS == 8) {
            uint32_t w0 = 0, w1 = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                w0 = __builtin_amdgcn_alignbit(f[j], w0, BITS);
                w1 = __builtin_amdgcn_alignbit(f[4 + j], w1, BITS);
            }
            if constexpr (BITS == 7) { w0 >>= 4; w1 >>= 4; }     // 28 bits used
            if (live) {
                sh_w[(2 * L.chunk) * wp + r] = w0;
                sh_w[(2 * L.chunk + 1) * wp + r] = w1;
            }
        }
    }
}

template <int BITS, bool SIMPLE>
__device__ inline void stage_codes(const QuantPackArgs &a, const Unit &U, const Bounds &B, const uint4 (&v)[QP_ITEMS],
                                   const Lane &L, int slot, const float *sh_s, const float *sh_y,
                                   float (&s8)[8], float (&y8)[8], int cur, bool fast, uint8_t *sh_codes, int pitch) {
    constexpr uint32_t MASK = (1u << BITS) - 1u;
#pragma unroll
    for (int k = 0; k < QP_ITEMS; ++k) {
        const int r = L.rr * QP_ITEMS + k;
        if (L.active && r < U.n) {
            uint32_t f[8];
            item_codes<SIMPLE>(a, U, B, v[k], L, r, slot, sh_s, sh_y, s8, y8, cur, fast, f);
            uint8_t *dst = sh_codes + r * pitch + 8 * L.chunk;
            *reinterpret_cast<uint32_t *>(dst) =
                (f[0] & MASK) | ((f[1] & MASK) << 8) | ((f[2] & MASK) << 16) | ((f[3] & MASK) << 24);
            *reinterpret_cast<uint32_t *>(dst + 4) =
                (f[4] & MASK) | ((f[5] & MASK) << 8) | ((f[6] & MASK) << 16) | ((f[7] & MASK) << 24);
        }
    }
}

// Store the staged words sh_w[plane * wp + row] of unit U, consecutive lanes
// on consecutive tokens of a plane. When a plane's rows fit the work-group a
// thread keeps one row and steps over planes, with several LDS reads in
// flight before their stores.
__device__ inline void store_words(const QuantPackArgs &a, const Unit &U, const uint32_t *sh_w, int wp, int tshift) {
    const int tid = threadIdx.x;
    const int span = 1 << tshift;
    if (span <= QP_THREADS) {
        const int r = tid & (span - 1);
        if (r >= U.n) return;
        const int P = QP_THREADS >> tshift;
        int w = tid >> tshift;
        const uint32_t *src = sh_w + w * wp + r;
        uint32_t *dst = word_at(a, U, w, r);
        const int sstep = P * wp;
        const int64_t gstep = (int64_t)P * a.L_cap;
#pragma unroll 4
        for (; w < a.W; w += P) {
            *dst = *src;
            src += sstep;
            dst += gstep;
        }
    } else {
        // more rows than threads: rows tid, tid + QP_THREADS, ... of every plane
        for (int r = tid; r < U.n; r += QP_THREADS) {
            const uint32_t *src = sh_w + r;
            uint32_t *dst = word_at(a, U, 0, r);
#pragma unroll 4
            for (int w = 0; w < a.W; ++w) {
                *dst = *src;
                src += wp;
                dst += a.L_cap;
            }
        }
    }
}

// Quantize and store unit U (rows in v) with the scales of LDS slot `slot`
// (packs: slot = local block). pack_fast: every scale of the unit is known to
// allow the division-free quotient. Ends with a barrier, after which LDS may
// be rewritten.
template <int BITS>
__device__ inline void quantize_unit(const QuantPackArgs &a, const Unit &U, const Bounds &B, const uint4 (&v)[QP_ITEMS],
                                     const Lane &L, int slot, const float *sh_s, const float *sh_y,
                                     uint8_t *sh_codes, bool pack_fast = false) {
    constexpr int CPW = 32 / BITS;
    const int tid = threadIdx.x;
    const int D = a.D;
    // a lane's 8 fields form whole words only at 4, 7 and 8 bits (a 2-bit word
    // would need a lane pair, whose shuffle costs more registers than staging)
    constexpr bool direct = (BITS == 4 || BITS == 7 || BITS == 8);

    // wave-uniform choice of the common path: one block, every scale of the
    // wave's channels allows the division-free quotient
    float s8[8], y8[8];
    bool fast = true;
    if (U.nb == 1 && L.active) fast = load_sy(sh_s, sh_y, slot, L, s8, y8);
    const bool simple = U.nb == 1 && __all(fast);
    const int cur = U.nb == 1 ? slot : -1;

    const int tshift = a.rows_log2;
    const int span = 1 << tshift;
    if constexpr (direct) {
        // words -> LDS planes -> global, consecutive lanes on consecutive
        // tokens of a plane. Odd plane pitch T + 1: the lanes of a wave (chunks
        // x rows 8 apart) then write distinct banks.
        uint32_t *sh_w = reinterpret_cast<uint32_t *>(sh_codes);
        const int wp = a.chunk_rows + 1;
        if (simple) stage_words<BITS, QM_SIMPLE>(a, U, B, v, L, slot, sh_s, sh_y, s8, y8, cur, fast, sh_w, wp);
        else if (U.nb > 1 && pack_fast) stage_words<BITS, QM_PACK>(a, U, B, v, L, slot, sh_s, sh_y, s8, y8, cur, fast, sh_w, wp);
        else stage_words<BITS, QM_GENERIC>(a, U, B, v, L, slot, sh_s, sh_y, s8, y8, cur, fast, sh_w, wp);
        lds_barrier();
        store_words(a, U, sh_w, wp, tshift);
        lds_barrier();
        return;
    }

    // ---- fields -> LDS code rows -> words, one plane at a time
    const int pitch = D >= 64 ? D + 4 : D;
    if (simple) stage_codes<BITS, true>(a, U, B, v, L, slot, sh_s, sh_y, s8, y8, cur, fast, sh_codes, pitch);
    else stage_codes<BITS, false>(a, U, B, v, L, slot, sh_s, sh_y, s8, y8, cur, fast, sh_codes, pitch);
    lds_barrier();
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
        *word_at(a, U, w, r) = word;
    }
    lds_barrier();
}

__device__ inline uint64_t tagged(uint32_t epoch, float m) { return ((uint64_t)epoch << 32) | f2u(m); }

__device__ inline uint64_t load_slot(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The maximum held by slot p, whose last load returned v, once the slot
// carries `epoch` (spins until then; a timeout is recorded in *status).
__device__ inline float slot_max(const uint64_t *p, uint64_t v, uint32_t epoch, uint32_t *status) {
    unsigned spins = 0;
    while ((uint32_t)(v >> 32) != epoch) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > QP_SPIN_LIMIT) {
            __hip_atomic_store(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        v = load_slot(p);
    }
    return u2f((uint32_t)v);
}

constexpr int QP_GATHER = 16;                                 // partial-maximum loads in flight per thread

// Per-channel maximum of the partial maxima of a block's n chunks, whose
// slots are the n * D consecutive words at p (chunk-major), by the whole
// work-group: thread t takes words t, t + QP_THREADS, ... with QP_GATHER loads
// in flight, and merges each into gx[channel] with an LDS max-atomic (the
// maxima are non-negative, so their bit patterns order like the values). gx
// must hold zeros, ordered before this call by a barrier; the caller orders
// the atomics before reading gx with another.
__device__ inline void gather_block_max(const uint64_t *p, int n, int D, uint32_t *gx, uint32_t epoch,
                                        uint32_t *status) {
    const int total = n * D;
    const int step = QP_THREADS % D;           // channel advance from word i to word i + QP_THREADS
    int ch = threadIdx.x % D;                  // channel of the next word merged
    for (int i0 = threadIdx.x; i0 < total; i0 += QP_GATHER * QP_THREADS) {
        uint64_t v[QP_GATHER];
#pragma unroll
        for (int j = 0; j < QP_GATHER; ++j) {
            const int i = i0 + j * QP_THREADS;
            if (i < total) v[j] = load_slot(p + i);
        }
#pragma unroll
        for (int j = 0; j < QP_GATHER; ++j) {
            const int i = i0 + j * QP_THREADS;
            if (i < total) atomicMax(gx + ch, f2u(slot_max(p + i, v[j], epoch, status)));
            ch += step;
            if (ch >= D) ch -= D;
        }
    }
}

// Scale and reciprocal of maximum m into LDS slot `slot` (thread = channel).
template <int BITS>
__device__ inline float put_scale(float *sh_s, float *sh_y, int slot, int D, int tid, float m) {
    constexpr float QMAX = (float)((1 << (BITS - 1)) - 1);
    const float s = m / QMAX;                                       // IEEE fp32 division
    sh_s[slot * D + tid] = s;
    sh_y[slot * D + tid] = recip_for_codes(s);
    return s;
}

// Row of the block maxima exchanged for block g0 of unit U: [tensor][b*H + h][block].
__device__ inline int64_t fin_row(const QuantPackArgs &a, const Unit &U) {
    return ((int64_t)U.t * a.B * a.H + U.bh) * a.G + U.g0;
}

__device__ inline float *scale_ptr(const QuantPackArgs &a, const Unit &U, int tid) {
    return (U.t ? a.scales2 : a.scales) + (U.bh * a.G_cap + a.group_start + U.g0) * a.D + tid;
}

// Channel tid of the block maximum merged in gx for last chunk U: published
// for the block's other chunks, stored as the block's scale and put in LDS
// slot R (whose scale row is gx itself; each thread reads its word first).
template <int BITS>
__device__ inline void publish_block_max(const QuantPackArgs &a, const Unit &U, float *sh_s, float *sh_y,
                                         const uint32_t *gx, uint32_t epoch) {
    const int tid = threadIdx.x;
    const float m = u2f(gx[tid]);
    __hip_atomic_store(a.fin + fin_row(a, U) * a.D + tid, tagged(epoch, m), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    *scale_ptr(a, U, tid) = put_scale<BITS>(sh_s, sh_y, QP_SLOT_R, a.D, tid, m);
}

// SPLIT: some block of this launch spans several units (exchange through
// scratch, cooperative launch). Otherwise every unit holds whole blocks and a
// work-group just quantizes its units one after another. LDS is sized by the
// host for this launch (regions at byte offsets a.lds_*). At most 128 VGPRs
// (four waves per SIMD), so that four work-groups share a CU.
template <int BITS, bool SPLIT>
__global__ __launch_bounds__(QP_THREADS) __attribute__((amdgpu_waves_per_eu(4))) void quant_pack_kernel(const QuantPackArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t qp_lds[];
    uint32_t *sh_max = reinterpret_cast<uint32_t *>(qp_lds + a.lds_max);   // [QP_MAX_PACK][D]
    float *sh_s = reinterpret_cast<float *>(qp_lds + a.lds_s);             // [QP_MAX_PACK + 2][D]
    float *sh_y = reinterpret_cast<float *>(qp_lds + a.lds_y);             // [QP_MAX_PACK + 2][D]
    uint8_t *sh_codes = qp_lds + a.lds_codes;                              // code rows or word planes
    int32_t *sh_off = reinterpret_cast<int32_t *>(qp_lds + a.lds_off);     // [G + 1]
    int32_t *sh_us = reinterpret_cast<int32_t *>(qp_lds + a.lds_us);       // [G + 1]

    const int tid = threadIdx.x;
    const int D = a.D;
    for (int i = tid; i <= a.G; i += QP_THREADS) {
        sh_off[i] = a.off[i];
        sh_us[i] = a.unit_start[i];
    }
    Lane L;
    L.tb.off = sh_off;
    L.tb.us = sh_us;
    L.D = D;
    L.lpr = D >> 3;
    L.RP = QP_THREADS / L.lpr;
    L.chunk = tid % L.lpr;
    L.rr = tid / L.lpr;
    L.active = L.rr < L.RP;
    L.xoff = (uint32_t)(8 * L.chunk) * 2u;
    const int64_t step = gridDim.x;
    for (int i = tid; i < QP_MAX_PACK * D; i += QP_THREADS) sh_max[i] = 0;

    if constexpr (!SPLIT) {
        // set when a scale of the current unit needs IEEE division
        __shared__ uint32_t sh_slow;
        lds_barrier();
        for (int64_t u = blockIdx.x; u < a.n_units; u += step) {
            const Unit U = unit_of(a, L.tb, u);
            uint4 X[QP_ITEMS];
            load_unit(a, U, X, L);
            const Bounds B = bounds_of(L.tb, U);
            if (tid == 0) sh_slow = 0;
            unit_absmax(a, U, B, X, L, sh_max);
            lds_barrier();
            // scales of the unit's blocks, (block, channel) pairs over all threads
            float *scl = scale_ptr(a, U, 0);
            for (int i = tid; i < U.nb * D; i += QP_THREADS) {
                const float m = u2f(sh_max[i]);
                sh_max[i] = 0;
                const int lb = i / D, c = i - lb * D;
                const float sc = put_scale<BITS>(sh_s, sh_y, lb, D, c, m);
                scl[i] = sc;
                if (!fast_scale_ok(sc)) sh_slow = 1;
            }
            lds_barrier();
            quantize_unit<BITS>(a, U, B, X, L, 0, sh_s, sh_y, sh_codes, sh_slow == 0);
        }
        return;
    }

    uint32_t *status = a.sync + 2;
    // Relaxed atomics suffice for the epoch word: the previous launch's write
    // is ordered before this launch by the stream, and every work-group reads
    // the word before its own increment below, so the work-group making the
    // last increment finds every read of this launch done. (Acquire and
    // acq_rel orderings here would cost a whole-L2 invalidate and write-back
    // per work-group.)
    uint32_t epoch = __hip_atomic_load(a.sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    if (epoch == 0) epoch = 1;
    lds_barrier();

    // Per unit: absmax; a chunk of a split block publishes its partial. The
    // block's last chunk gathers every partial, publishes the block maximum
    // and is quantized; any other chunk waits for that maximum and is
    // quantized. Units of whole blocks are quantized at once. Only the
    // current unit is held in registers.
    uint32_t *gx = reinterpret_cast<uint32_t *>(sh_y + QP_SLOT_R * D);   // gather row (slot R)
    for (int64_t u = blockIdx.x; u < a.n_units; u += step) {
        const Unit U = unit_of(a, L.tb, u);
        uint4 X[QP_ITEMS];
        load_unit(a, U, X, L);
        const Bounds B = bounds_of(L.tb, U);
        const bool split = U.nc > 1, last = split && U.c == U.nc - 1;
        // slot R's rows were last read before the previous unit's final barrier
        if (last && tid < D) gx[tid] = 0;
        unit_absmax(a, U, B, X, L, sh_max);
        lds_barrier();
        if (tid < D) {
            const float m0 = u2f(sh_max[tid]);
            sh_max[tid] = 0;
            if (split) {
                __hip_atomic_store(a.part + U.id * D + tid, tagged(epoch, m0), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            } else {
                // whole blocks: scales now; block maxima in LDS are cleared
                // for the next unit (ordered before its atomics by the barrier)
                float *scl = scale_ptr(a, U, tid);
                for (int lb = 0; lb < U.nb; ++lb) {
                    float m = m0;
                    if (lb > 0) {
                        m = u2f(sh_max[lb * D + tid]);
                        sh_max[lb * D + tid] = 0;
                    }
                    scl[(int64_t)lb * D] = put_scale<BITS>(sh_s, sh_y, lb, D, tid, m);
                }
            }
        }
        int slot = 0;
        if (last) {
            gather_block_max(a.part + (U.id - U.c) * D, U.nc, D, gx, epoch, status);
            lds_barrier();
            if (tid < D) publish_block_max<BITS>(a, U, sh_s, sh_y, gx, epoch);
            slot = QP_SLOT_R;
        } else if (split) {
            if (tid < D) {
                const uint64_t *fin = a.fin + fin_row(a, U) * D + tid;
                put_scale<BITS>(sh_s, sh_y, QP_SLOT_W, D, tid, slot_max(fin, load_slot(fin), epoch, status));
            }
            slot = QP_SLOT_W;
        }
        lds_barrier();
        quantize_unit<BITS>(a, U, B, X, L, slot, sh_s, sh_y, sh_codes);
    }

    // ---- the last work-group to finish advances the epoch for the next launch
    if (tid == 0) {
        const uint32_t done = __hip_atomic_fetch_add(a.sync + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {
            __hip_atomic_store(a.sync + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.sync, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------- slab kernel
//
// Blocks longer than one unit, without any exchange between work-groups: a
// work-group owns one (tensor, batch, head, block) and SW consecutive channels
// (a slab) for ALL the block's rows, so each channel's absmax is complete
// inside it. Thread (r0, q) holds channels [8q, 8q + 8) of the slab in rows
// r0, r0 + RS, ..., RPT rows (RS = NT / (SW / 8) rows per step, NT = 512 or
// 1024 threads); all its row loads are issued at once, rows past the block
// re-read its last row. The
// maxima are reduced across the lanes of a wave that share q, then across
// waves with LDS max-atomics; each channel's scale s = fp32(m / qmax) is
// stored, and the codes (the same division-free exact quotient as the unit
// kernel) are packed in registers: at 4 bits a lane's 8 channels are one
// word, at 7 and 8 bits two, at 2 bits a lane pair's 16 channels one word.
// Packing needs whole words inside a slab: BITS in {2, 4, 7, 8}.

template <int BITS, int SW, int RPT, int NT>
__global__ __launch_bounds__(NT) void quant_slab_kernel(const SlabArgs a) {
    static_assert(BITS == 2 || BITS == 4 || BITS == 7 || BITS == 8, "whole words per slab");
    static_assert(SW % 16 == 0, "slabs of 16 or 32 channels");
    constexpr int LPR = SW / 8;                    // threads per row
    constexpr int RS = NT / LPR;                   // rows per step
    constexpr float QMAX = (float)((1 << (BITS - 1)) - 1);
    __shared__ uint32_t sh_max[SW];
    __shared__ __attribute__((aligned(16))) float sh_s[SW];
    __shared__ __attribute__((aligned(16))) float sh_y[SW];
    __shared__ uint32_t sh_slow;

    const int64_t lid = xcd_logical_id(blockIdx.x, a.n_units);
    if (lid < 0) return;
    // logical id = (((t * B*H + bh) * nbig + j) * slabs + c), largest blocks
    // (the last ones) first; the slabs of one block run side by side
    const int c = (int)(lid % a.slabs);
    int64_t v = lid / a.slabs;
    const int jr = (int)(v % a.nbig);
    v /= a.nbig;
    const int bh = (int)(v % ((int64_t)a.B * a.H));
    const int t = (int)(v / ((int64_t)a.B * a.H));
    const int g = a.gb + (a.nbig - 1 - jr);
    const int row0 = a.off[g], n = a.off[g + 1] - row0;
    const int b = bh / a.H, h = bh % a.H;

    const int tid = threadIdx.x;
    const int q = tid % LPR, r0 = tid / LPR;
    if (tid < SW) sh_max[tid] = 0;
    if (tid == 0) sh_slow = 0;

    // ---- all row loads in flight at once
    const uint16_t *x = a.x[t] + (int64_t)b * a.sx_b[t] + (int64_t)h * a.sx_h[t] + (int64_t)row0 * a.sx_l[t] +
                        c * SW + 8 * q;
    // the row stride in bytes fits 32 bits (the host checks), so a row address
    // is one 32 x 32 -> 64-bit multiply-add
    const char *xb = reinterpret_cast<const char *>(x);
    const uint32_t slb = (uint32_t)a.sx_l[t] * 2u;
    uint4 xv[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        const uint32_t r = (uint32_t)min(r0 + k * RS, n - 1);
        xv[k] = *reinterpret_cast<const uint4 *>(xb + (uint64_t)r * slb);
    }

    // ---- absmax: packed 16-bit maxima of |x| (bf16 patterns with the sign
    // cleared order like the values), reduced over the lanes sharing q
    u16x2 m[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = u16x2{0, 0};
#pragma unroll
    for (int k = 0; k < RPT; ++k) absmax_item(m, xv[k]);
#pragma unroll
    for (int d = LPR; d < 64; d <<= 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t o = __shfl_xor(__builtin_bit_cast(uint32_t, m[j]), d);
            m[j] = __builtin_elementwise_max(m[j], __builtin_bit_cast(u16x2, o));
        }
    }
    lds_barrier();                                 // sh_max cleared
    if ((tid & 63) < LPR) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t w = __builtin_bit_cast(uint32_t, m[j]);
            atomicMax(&sh_max[8 * q + 2 * j], w << 16);
            atomicMax(&sh_max[8 * q + 2 * j + 1], w & 0xFFFF0000u);
        }
    }
    lds_barrier();

    // ---- scales of the slab's channels
    if (tid < SW) {
        const float mx = u2f(sh_max[tid]);
        const float s = mx / QMAX;                 // IEEE fp32 division
        sh_s[tid] = s;
        sh_y[tid] = recip_for_codes(s);
        a.scales[t][((int64_t)bh * a.G_cap + a.group_start + g) * a.D + c * SW + tid] = s;
        if (!fast_scale_ok(s)) sh_slow = 1;
    }
    lds_barrier();

    // ---- codes and words
    float s8[8], y8[8];
    {
        const float4 *ps = reinterpret_cast<const float4 *>(sh_s + 8 * q);
        const float4 *py = reinterpret_cast<const float4 *>(sh_y + 8 * q);
        const float4 s0 = ps[0], s1 = ps[1], y0 = py[0], y1 = py[1];
        s8[0] = s0.x; s8[1] = s0.y; s8[2] = s0.z; s8[3] = s0.w; s8[4] = s1.x; s8[5] = s1.y; s8[6] = s1.z; s8[7] = s1.w;
        y8[0] = y0.x; y8[1] = y0.y; y8[2] = y0.z; y8[3] = y0.w; y8[4] = y1.x; y8[5] = y1.y; y8[6] = y1.z; y8[7] = y1.w;
    }
    const bool fast = __builtin_amdgcn_readfirstlane(sh_slow) == 0;
    constexpr int CPW = 32 / BITS;
    const int ch0 = c * SW + 8 * q;                // the lane's first channel
    // the lane's word plane from its first row on; row r0 + k * RS is then a
    // constant offset
    uint32_t *pw = a.packed[t] + ((int64_t)bh * a.W + ch0 / CPW) * a.L_cap + a.tok_start + row0 + r0;
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        const int r = r0 + k * RS;
        uint32_t f[8];
        if (fast) codes8<true>(xv[k], s8, y8, f);
        else codes8<false>(xv[k], s8, y8, f);
        // fields enter a word from the top (alignbit keeps the low BITS bits)
        if constexpr (BITS == 4) {
            uint32_t w = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) w = __builtin_amdgcn_alignbit(f[j], w, 4);
            if (r < n) pw[k * RS] = w;
        } else if constexpr (BITS == 7 || BITS == 8) {
            uint32_t w0 = 0, w1 = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                w0 = __builtin_amdgcn_alignbit(f[j], w0, BITS);
                w1 = __builtin_amdgcn_alignbit(f[4 + j], w1, BITS);
            }
            if constexpr (BITS == 7) { w0 >>= 4; w1 >>= 4; }     // 28 bits used
            if (r < n) {
                pw[k * RS] = w0;
                pw[a.L_cap + k * RS] = w1;
            }
        } else {
            // 2 bits: this lane's 8 fields are one half of a 16-channel word;
            // the even lane of the pair (channels 16p .. 16p + 15) stores it
            uint32_t w = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) w = __builtin_amdgcn_alignbit(f[j], w, 2);
            const uint32_t half = w >> 16;
            const uint32_t other = __shfl_xor(half, 1);
            if ((q & 1) == 0 && r < n) pw[k * RS] = half | (other << 16);
        }
    }
}

// Slab width at 3, 5 and 6 bits: the least multiple of 8 channels (one lane's
// 16-byte load) that is also a multiple of the codes per word (10, 6, 5), so
// every slab starts on a word boundary; the last slab of a row takes the
// remaining D mod width channels (a multiple of 8, whole words up to the row's
// last, partial word).
constexpr int staged_slab_width(int bits) { return bits == 5 ? 24 : 40; }

// quantize+pack of whole long blocks at 3, 5 or 6 bits, one work-group per
// (tensor, batch, head, block, slab), with no exchange: words straddle the
// lanes' 8-channel loads, so the codes go through LDS as bytes ([row][slab]
// in dynamic LDS, rows * width bytes) and words are assembled from there.
template <int BITS, int RPT, int NT>
__global__ __launch_bounds__(NT) void quant_slab_staged_kernel(const SlabArgs a) {
    static_assert(BITS == 3 || BITS == 5 || BITS == 6, "codes straddle the lanes' channel octets");
    constexpr int CPW = 32 / BITS;
    constexpr int SW = staged_slab_width(BITS);
    constexpr int WSMAX = (SW + CPW - 1) / CPW;
    constexpr float QMAX = (float)((1 << (BITS - 1)) - 1);
    extern __shared__ __attribute__((aligned(16))) uint8_t sh_codes[];
    __shared__ uint32_t sh_max[SW];
    __shared__ __attribute__((aligned(16))) float sh_s[SW];
    __shared__ __attribute__((aligned(16))) float sh_y[SW];
    __shared__ uint32_t sh_slow;

    const int64_t lid = xcd_logical_id(blockIdx.x, a.n_units);
    if (lid < 0) return;
    const int c = (int)(lid % a.slabs);
    int64_t v = lid / a.slabs;
    const int jr = (int)(v % a.nbig);
    v /= a.nbig;
    const int bh = (int)(v % ((int64_t)a.B * a.H));
    const int t = (int)(v / ((int64_t)a.B * a.H));
    const int g = a.gb + (a.nbig - 1 - jr);
    const int row0 = a.off[g], n = a.off[g + 1] - row0;
    const int b = bh / a.H, h = bh % a.H;

    const int ch0 = c * SW;
    const int width = min(SW, a.D - ch0);          // a multiple of 8
    const int lpr = width >> 3;                    // lanes per row
    const int rs = NT / lpr;                       // rows per step
    const int steps = (n + rs - 1) / rs;           // <= RPT (checked on the host)
    const int tid = threadIdx.x;
    const int q = tid % lpr, r0 = tid / lpr;
    const bool active = r0 < rs;
    if (tid < SW) sh_max[tid] = 0;
    if (tid == 0) sh_slow = 0;

    // ---- all row loads in flight at once (rows past n re-read row n - 1)
    const uint16_t *x = a.x[t] + (int64_t)b * a.sx_b[t] + (int64_t)h * a.sx_h[t] + (int64_t)row0 * a.sx_l[t] +
                        ch0 + 8 * q;
    // the row stride in bytes fits 32 bits (the host checks)
    const char *xb = reinterpret_cast<const char *>(x);
    const uint32_t slb = (uint32_t)a.sx_l[t] * 2u;
    uint4 xv[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        xv[k] = make_uint4(0, 0, 0, 0);
        if (active && k < steps) {
            const uint32_t r = (uint32_t)min(r0 + k * rs, n - 1);
            xv[k] = *reinterpret_cast<const uint4 *>(xb + (uint64_t)r * slb);
        }
    }

    // ---- absmax per channel: the lane's rows, then LDS max-atomics
    u16x2 m[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] = u16x2{0, 0};
#pragma unroll
    for (int k = 0; k < RPT; ++k)
        if (k < steps) absmax_item(m, xv[k]);      // zero for inactive lanes
    lds_barrier();                                 // sh_max cleared
    if (active) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t w = __builtin_bit_cast(uint32_t, m[j]);
            atomicMax(&sh_max[8 * q + 2 * j], w << 16);
            atomicMax(&sh_max[8 * q + 2 * j + 1], w & 0xFFFF0000u);
        }
    }
    lds_barrier();

    // ---- scales of the slab's channels
    if (tid < width) {
        const float mx = u2f(sh_max[tid]);
        const float sc = mx / QMAX;                // IEEE fp32 division
        sh_s[tid] = sc;
        sh_y[tid] = recip_for_codes(sc);
        a.scales[t][((int64_t)bh * a.G_cap + a.group_start + g) * a.D + ch0 + tid] = sc;
        if (!fast_scale_ok(sc)) sh_slow = 1;
    }
    lds_barrier();

    // ---- codes as bytes into LDS, row r of the slab at r * SW
    if (active) {
        float s8[8], y8[8];
        const float4 *ps = reinterpret_cast<const float4 *>(sh_s + 8 * q);
        const float4 *py = reinterpret_cast<const float4 *>(sh_y + 8 * q);
        const float4 s0 = ps[0], s1 = ps[1], y0 = py[0], y1 = py[1];
        s8[0] = s0.x; s8[1] = s0.y; s8[2] = s0.z; s8[3] = s0.w; s8[4] = s1.x; s8[5] = s1.y; s8[6] = s1.z; s8[7] = s1.w;
        y8[0] = y0.x; y8[1] = y0.y; y8[2] = y0.z; y8[3] = y0.w; y8[4] = y1.x; y8[5] = y1.y; y8[6] = y1.z; y8[7] = y1.w;
        const bool fast = __builtin_amdgcn_readfirstlane(sh_slow) == 0;
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
            const int r = r0 + k * rs;
            if (k < steps && r < n) {
                uint32_t f[8];
                if (fast) codes8<true>(xv[k], s8, y8, f);
                else codes8<false>(xv[k], s8, y8, f);
                const uint32_t lo = (f[0] & 0xFFu) | ((f[1] & 0xFFu) << 8) | ((f[2] & 0xFFu) << 16) | (f[3] << 24);
                const uint32_t hi = (f[4] & 0xFFu) | ((f[5] & 0xFFu) << 8) | ((f[6] & 0xFFu) << 16) | (f[7] << 24);
                *reinterpret_cast<uint2 *>(sh_codes + r * SW + 8 * q) = make_uint2(lo, hi);
            }
        }
    }
    lds_barrier();

    // ---- words: word wi of the slab holds its codes wi*CPW .. (from the low
    // bits up); consecutive threads take consecutive rows of one word plane
    const int ws = (width + CPW - 1) / CPW;
    uint32_t *pk = a.packed[t] + ((int64_t)bh * a.W + ch0 / CPW) * a.L_cap + a.tok_start + row0;
#pragma unroll
    for (int wi = 0; wi < WSMAX; ++wi) {
        if (wi >= ws) break;
        const int start = wi * CPW;                // first code byte of the word in the row
        const int nc = min(CPW, width - start);
        const int base8 = start & ~7, off = start & 7;
        for (int r = tid; r < n; r += NT) {
            const uint8_t *row = sh_codes + r * SW + base8;
            const uint2 lo = *reinterpret_cast<const uint2 *>(row);
            const uint2 hi = (off + CPW > 8) ? *reinterpret_cast<const uint2 *>(row + 8) : make_uint2(0, 0);
            const uint32_t d[4] = {lo.x, lo.y, hi.x, hi.y};
            uint32_t w = 0;
#pragma unroll
            for (int j = 0; j < CPW; ++j) {
                const int byte = off + j;
                if (j < nc) w |= __builtin_amdgcn_ubfe(d[byte >> 2], 8 * (byte & 3), BITS) << (BITS * j);
            }
            pk[(int64_t)wi * a.L_cap + r] = w;
        }
    }
}

// Rows of one block that a slab work-group of nt threads holds at sw
// channels per slab (16 row steps per thread).
int quant_slab_max_rows(int sw, int nt) { return (nt / (sw / 8)) * 16; }

template <int BITS, int SW, int NT>
static hipError_t launch_slab_nt(const SlabArgs &a, int rpt, hipStream_t st) {
    const int64_t grid = (a.n_units + 7) / 8 * 8;
    if (rpt <= 4)
        hipLaunchKernelGGL((quant_slab_kernel<BITS, SW, 4, NT>), dim3((unsigned)grid), dim3(NT), 0, st, a);
    else if (rpt <= 8)
        hipLaunchKernelGGL((quant_slab_kernel<BITS, SW, 8, NT>), dim3((unsigned)grid), dim3(NT), 0, st, a);
    else if (rpt <= 16)
        hipLaunchKernelGGL((quant_slab_kernel<BITS, SW, 16, NT>), dim3((unsigned)grid), dim3(NT), 0, st, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int BITS, int SW>
static hipError_t launch_slab_sw(const SlabArgs &a, int rpt, int nt, hipStream_t st) {
    if (nt == 256) return launch_slab_nt<BITS, SW, 256>(a, rpt, st);
    if (nt == 512) return launch_slab_nt<BITS, SW, 512>(a, rpt, st);
    if (nt == 1024) return launch_slab_nt<BITS, SW, 1024>(a, rpt, st);
    return hipErrorInvalidValue;
}

template <int BITS>
static hipError_t launch_slab_bits(const SlabArgs &a, int sw, int rpt, int nt, hipStream_t st) {
    if (sw == 32) return launch_slab_sw<BITS, 32>(a, rpt, nt, st);
    if (sw == 16) return launch_slab_sw<BITS, 16>(a, rpt, nt, st);
    return hipErrorInvalidValue;
}

// Rows of one block that a staged slab work-group of nt threads holds at 3,
// 5 or 6 bits (16 row steps per thread of the full slab width, and the codes
// of every row in 63 KB of dynamic LDS, within the 64 KB a launch gets
// without an attribute).
int quant_slab_staged_max_rows(int bits, int nt) {
    const int sw = staged_slab_width(bits);
    return std::min((nt / (sw / 8)) * 16, 64512 / sw);
}

int quant_slab_staged_width(int bits) { return staged_slab_width(bits); }

template <int BITS, int NT>
static hipError_t launch_staged_nt(const SlabArgs &a, int rpt, int max_rows, hipStream_t st) {
    const int64_t grid = (a.n_units + 7) / 8 * 8;
    const size_t lds = (size_t)max_rows * staged_slab_width(BITS);
    if (rpt <= 4)
        hipLaunchKernelGGL((quant_slab_staged_kernel<BITS, 4, NT>), dim3((unsigned)grid), dim3(NT), lds, st, a);
    else if (rpt <= 8)
        hipLaunchKernelGGL((quant_slab_staged_kernel<BITS, 8, NT>), dim3((unsigned)grid), dim3(NT), lds, st, a);
    else if (rpt <= 16)
        hipLaunchKernelGGL((quant_slab_staged_kernel<BITS, 16, NT>), dim3((unsigned)grid), dim3(NT), lds, st, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int BITS>
static hipError_t launch_staged_bits(const SlabArgs &a, int rpt, int nt, int max_rows, hipStream_t st) {
    if (nt == 256) return launch_staged_nt<BITS, 256>(a, rpt, max_rows, st);
    if (nt == 512) return launch_staged_nt<BITS, 512>(a, rpt, max_rows, st);
    if (nt == 1024) return launch_staged_nt<BITS, 1024>(a, rpt, max_rows, st);
    return hipErrorInvalidValue;
}

// Staged slab launch (3, 5 or 6 bits) over the blocks [a.gb, a.gb + a.nbig),
// the longest of max_rows rows.
hipError_t launch_quant_slab_staged(const SlabArgs &a, int bits, int rpt, int nt, int max_rows, hipStream_t st) {
    switch (bits) {
        case 3: return launch_staged_bits<3>(a, rpt, nt, max_rows, st);
        case 5: return launch_staged_bits<5>(a, rpt, nt, max_rows, st);
        case 6: return launch_staged_bits<6>(a, rpt, nt, max_rows, st);
        default: return hipErrorInvalidValue;
    }
}

// Slab launch over the blocks [a.gb, a.gb + a.nbig) with sw channels per slab,
// nt threads per work-group and rpt row steps per thread
// (rows <= rpt * nt / (sw / 8)).
hipError_t launch_quant_slab(const SlabArgs &a, int bits, int sw, int rpt, int nt, hipStream_t st) {
    switch (bits) {
        case 2: return launch_slab_bits<2>(a, sw, rpt, nt, st);
        case 4: return launch_slab_bits<4>(a, sw, rpt, nt, st);
        case 7: return launch_slab_bits<7>(a, sw, rpt, nt, st);
        case 8: return launch_slab_bits<8>(a, sw, rpt, nt, st);
        default: return hipErrorInvalidValue;
    }
}

template <int BITS>
static hipError_t launch_qp(const QuantPackArgs &a, int grid, bool split, hipStream_t st) {
    if (!split) {
        hipLaunchKernelGGL((quant_pack_kernel<BITS, false>), dim3(grid), dim3(QP_THREADS), a.lds_bytes, st, a);
        return hipGetLastError();
    }
    void *args[] = {const_cast<QuantPackArgs *>(&a)};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void *>(&quant_pack_kernel<BITS, true>),
                                      dim3(grid), dim3(QP_THREADS), args, (unsigned)a.lds_bytes, st);
}

template <int BITS>
static int qp_resident_blocks(int lds_bytes) {
    int per_cu = 0, cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quant_pack_kernel<BITS, true>, QP_THREADS,
                                                     (size_t)lds_bytes) != hipSuccess)
        return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return per_cu * cus;
}

int quant_pack_unit_elems() { return QP_UNIT_ELEMS; }
int quant_pack_max_pack() { return QP_MAX_PACK; }

// Work-groups of the split kernel that fit the device at once, for this LDS
// size (cached per device, bit width and LDS size).
int quant_pack_resident_blocks(int bits, int lds_bytes) {
    struct Entry { int dev, bits, lds, n; };
    static Entry cache[64];
    static int used = 0;
    static std::mutex mu;
    int dev = 0;
    if (bits < 2 || bits > 8 || hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lk(mu);
    for (int i = 0; i < used; ++i)
        if (cache[i].dev == dev && cache[i].bits == bits && cache[i].lds == lds_bytes) return cache[i].n;
    int r = 0;
    switch (bits) {
        case 2: r = qp_resident_blocks<2>(lds_bytes); break;
        case 3: r = qp_resident_blocks<3>(lds_bytes); break;
        case 4: r = qp_resident_blocks<4>(lds_bytes); break;
        case 5: r = qp_resident_blocks<5>(lds_bytes); break;
        case 6: r = qp_resident_blocks<6>(lds_bytes); break;
        case 7: r = qp_resident_blocks<7>(lds_bytes); break;
        case 8: r = qp_resident_blocks<8>(lds_bytes); break;
    }
    if (r > 0 && used < 64) cache[used++] = Entry{dev, bits, lds_bytes, r};
    return r;
}

hipError_t launch_quant_pack(const QuantPackArgs &a, int bits, int grid, bool split, hipStream_t st) {
    switch (bits) {
        case 2: return launch_qp<2>(a, grid, split, st);
        case 3: return launch_qp<3>(a, grid, split, st);
        case 4: return launch_qp<4>(a, grid, split, st);
        case 5: return launch_qp<5>(a, grid, split, st);
        case 6: return launch_qp<6>(a, grid, split, st);
        case 7: return launch_qp<7>(a, grid, split, st);
        case 8: return launch_qp<8>(a, grid, split, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace varq
