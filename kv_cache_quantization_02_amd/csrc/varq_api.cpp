// varq_api.cpp - C ABI of the VAR-Q packed KV-cache library: argument
// validation, work decomposition and launches on the caller's stream.
// Nothing here computes on the host beyond sizes and launch tables; every step
// of quantization, packing and attention runs in the gfx950 kernels.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "../../include/varq.h"
#include "varq_device.h"

namespace varq {
hipError_t launch_quant_pack(const QuantPackArgs &a, int bits, int grid, bool split, hipStream_t st);
int quant_pack_resident_blocks(int bits, int lds_bytes);
int quant_pack_max_pack();
hipError_t launch_unpack_dequant(const UnpackArgs &a, int bits, hipStream_t st);
hipError_t launch_packed_attention(const AttnArgs &a, int D, int bits, hipStream_t st);
hipError_t launch_dense_attention(const AttnArgs &a, int D, hipStream_t st);
hipError_t launch_quant_group(const GroupArgs &a, int mode, int bits, int64_t n_scales, hipStream_t st);
int attention_q_tile();
}  // namespace varq

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return VARQ_OK;
}

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int check_bits(int bits) {
    if (bits < 2 || bits > 8) return fail(VARQ_EBITS, "bits must be in 2..8 (got %d)", bits);
    return VARQ_OK;
}

// group_offsets: host int32[G+1], 0 = o_0 < ... < o_G = L.
int check_offsets(const int32_t *off, int G, int64_t L, const char *what) {
    if (G < 1 || G > VARQ_MAX_GROUPS)
        return fail(VARQ_EINVAL, "%s: number of blocks G=%d outside 1..%d", what, G, VARQ_MAX_GROUPS);
    if (off == nullptr) return fail(VARQ_EINVAL, "%s: group_offsets is NULL", what);
    if (off[0] != 0) return fail(VARQ_EINVAL, "%s: group_offsets[0] must be 0 (got %d)", what, off[0]);
    for (int g = 0; g < G; ++g)
        if (off[g + 1] <= off[g])
            return fail(VARQ_EINVAL, "%s: group_offsets must strictly increase (o[%d]=%d, o[%d]=%d)",
                        what, g, off[g], g + 1, off[g + 1]);
    if ((int64_t)off[G] != L)
        return fail(VARQ_EINVAL, "%s: group_offsets[G] = %d must equal the token count %lld", what,
                    off[G], (long long)L);
    return VARQ_OK;
}

int launch_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(VARQ_ELAUNCH, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
    return ok();
}

int words_per_row(int D, int bits) {
    const int cpw = 32 / bits;
    return (D + cpw - 1) / cpw;
}

// Device scratch for quantize+pack's cross-work-group exchange, per (device,
// stream). `sync` (epoch, finished count, status) is allocated once and zeroed;
// the kernel leaves the count at zero and advances the epoch. `slots` grows on
// demand and is zeroed when allocated; afterwards every slot the kernel reads
// carries the epoch of the launch that wrote it, so stale contents never pass
// for current ones, whatever the shapes of earlier calls.
struct Scratch {
    uint32_t *sync = nullptr;
    uint64_t *slots = nullptr;
    size_t n_slots = 0;
    float *attn = nullptr;      // attention partials of KV-split launches
    size_t attn_bytes = 0;
};
std::mutex g_scratch_mu;
std::map<std::pair<int, hipStream_t>, Scratch> g_scratch;

int scratch_for(hipStream_t st, size_t n_slots, uint32_t **sync, uint64_t **slots) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(VARQ_ELAUNCH, "quantize_pack: no current device");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    Scratch &s = g_scratch[{dev, st}];
    if (!s.sync) {
        void *p = nullptr;
        if (hipMalloc(&p, 4 * sizeof(uint32_t)) != hipSuccess || hipMemset(p, 0, 4 * sizeof(uint32_t)) != hipSuccess)
            return fail(VARQ_ELAUNCH, "quantize_pack: scratch allocation failed");
        s.sync = static_cast<uint32_t *>(p);
    }
    if (s.n_slots < n_slots) {
        if (s.slots) {
            // the old buffer may still be in use by work queued on this stream
            if (hipStreamSynchronize(st) != hipSuccess || hipFree(s.slots) != hipSuccess)
                return fail(VARQ_ELAUNCH, "quantize_pack: cannot release scratch");
            s.slots = nullptr;
            s.n_slots = 0;
        }
        void *p = nullptr;
        if (hipMalloc(&p, n_slots * 8) != hipSuccess) return fail(VARQ_ELAUNCH, "quantize_pack: scratch allocation failed");
        if (hipMemset(p, 0, n_slots * 8) != hipSuccess) return fail(VARQ_ELAUNCH, "quantize_pack: scratch clear failed");
        s.slots = static_cast<uint64_t *>(p);
        s.n_slots = n_slots;
    }
    *sync = s.sync;
    *slots = s.slots;
    return VARQ_OK;
}


// Attention partials for a launch split over KV ranges, per (device, stream),
// grown on demand (after synchronizing that stream) and kept until the
// process ends. Every launch writes all the partials it reads.
int attn_scratch_for(hipStream_t st, size_t bytes, float **p_out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(VARQ_ELAUNCH, "packed_attention: no current device");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    Scratch &s = g_scratch[{dev, st}];
    if (s.attn_bytes < bytes) {
        if (s.attn) {
            if (hipStreamSynchronize(st) != hipSuccess || hipFree(s.attn) != hipSuccess)
                return fail(VARQ_ELAUNCH, "packed_attention: cannot release scratch");
            s.attn = nullptr;
            s.attn_bytes = 0;
        }
        void *p = nullptr;
        if (hipMalloc(&p, bytes) != hipSuccess) return fail(VARQ_ELAUNCH, "packed_attention: scratch allocation failed");
        s.attn = static_cast<float *>(p);
        s.attn_bytes = bytes;
    }
    *p_out = s.attn;
    return VARQ_OK;
}

int device_cus() {
    static std::mutex mu;
    static std::map<int, int> cus;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lk(mu);
    auto it = cus.find(dev);
    if (it != cus.end()) return it->second;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    cus[dev] = n;
    return n;
}

// Number of KV ranges for an attention launch of `wgs` work-groups over `nt`
// 64-token tiles: 1 when the grid fills at least two rounds of resident
// work-groups; otherwise the count (ranges of at least 8 tiles) that
// minimizes rounds x (tiles per range + 4), the 4 standing for a work-group's
// fixed cost (query load, first tile, output).
int plan_kv_splits(int64_t wgs, int nt, int per_cu) {
    const int cus = device_cus();
    if (cus <= 0) return 1;
    const int64_t slots = (int64_t)cus * per_cu;
    if (wgs >= 2 * slots) return 1;
    auto cost = [&](int S) {
        const int64_t rounds = (wgs * S + slots - 1) / slots;
        return rounds * ((nt + S - 1) / S + 4);
    };
    int best = 1;
    for (int S = 2; S <= varq::VARQ_MAX_KV_SPLITS && nt / S >= 8; ++S)
        if (cost(S) < cost(best)) best = S;
    return best;
}

// KV ranges of an attention launch (a.off, a.L_kv, a.Lq, a.B, a.H and
// a.n_qtiles set): one range, or the planned split with its partials scratch.
int setup_kv_ranges(varq::AttnArgs &a, int D, void *stream) {
    const int nt = (int)((a.L_kv + 63) / 64);
    a.kv_splits = 1;
    a.split_t0[0] = 0;
    a.split_t0[1] = nt;
    a.split_g0[0] = 0;
    const int S = plan_kv_splits((int64_t)a.n_qtiles * a.B * a.H, nt, D == 64 ? 2 : 1);
    if (S == 1) return VARQ_OK;
    a.kv_splits = S;
    int g = 0;
    for (int k = 0; k < S; ++k) {
        a.split_t0[k] = (int32_t)((int64_t)nt * k / S);
        while (a.off[g + 1] <= (int64_t)a.split_t0[k] * 64) ++g;
        a.split_g0[k] = g;
    }
    a.split_t0[S] = nt;
    const size_t rows = (size_t)S * a.B * a.H * a.Lq;
    float *part = nullptr;
    if (int r = attn_scratch_for(static_cast<hipStream_t>(stream), rows * (D + 2) * sizeof(float), &part)) return r;
    a.part_o = part;
    a.part_ml = part + rows * D;
    return VARQ_OK;
}

// Validates one tensor's quantize+pack arguments and fills the launch
// arguments; *empty is set when there is nothing to write.
int qp_setup(const void *x, int64_t sx_b, int64_t sx_l, int64_t sx_h,
             int B, int H, int D, int64_t L_in,
             const int32_t *group_offsets, int G_in, int bits,
             int32_t *packed, int64_t L_cap, int64_t tok_start,
             float *scales, int64_t G_cap, int64_t group_start,
             varq::QuantPackArgs &a, bool *empty, bool *split, int *max_chunks) {
    *empty = false;
    if (int r = check_bits(bits)) return r;
    if (B < 1 || H < 1) return fail(VARQ_EINVAL, "quantize_pack: B=%d H=%d must be >= 1", B, H);
    if (D < 8 || D > 256 || D % 8 != 0)
        return fail(VARQ_EINVAL, "quantize_pack: head_dim %d must be a multiple of 8 in 8..256", D);
    if (L_in < 0) return fail(VARQ_EINVAL, "quantize_pack: L_in=%lld < 0", (long long)L_in);
    if (L_in == 0 && G_in == 0) { *empty = true; return ok(); }    // nothing to write
    if (int r = check_offsets(group_offsets, G_in, L_in, "quantize_pack")) return r;
    if (!x || !packed || !scales) return fail(VARQ_EINVAL, "quantize_pack: NULL tensor pointer");
    if (!aligned(x, 16) || sx_b % 8 || sx_l % 8 || sx_h % 8)
        return fail(VARQ_EALIGN, "quantize_pack: x must be 16-byte aligned with strides that are multiples of 8");
    if (!aligned(packed, 16) || L_cap % 8)
        return fail(VARQ_EALIGN, "quantize_pack: packed must be 16-byte aligned and L_cap a multiple of 8");
    if (!aligned(scales, 4)) return fail(VARQ_EALIGN, "quantize_pack: scales must be 4-byte aligned");
    if (tok_start < 0 || group_start < 0 || tok_start + L_in > L_cap || group_start + G_in > G_cap)
        return fail(VARQ_ECAPACITY,
                    "quantize_pack: rows [%lld, %lld) / blocks [%lld, %lld) exceed the cache (L_cap=%lld, G_cap=%lld)",
                    (long long)tok_start, (long long)(tok_start + L_in), (long long)group_start,
                    (long long)(group_start + G_in), (long long)L_cap, (long long)G_cap);

    std::memset(&a, 0, sizeof(a));
    a.x = static_cast<const uint16_t *>(x);
    a.sx_b = sx_b; a.sx_l = sx_l; a.sx_h = sx_h;
    a.packed = reinterpret_cast<uint32_t *>(packed);
    a.scales = scales;
    a.L_cap = L_cap; a.tok_start = tok_start; a.G_cap = G_cap; a.group_start = group_start;
    a.B = B; a.H = H; a.D = D; a.G = G_in;
    a.W = words_per_row(D, bits);
    // Units of at most T rows (T * D = the elements one work-group holds): a
    // block longer than T is cut into chunks; shorter consecutive blocks are
    // packed together, up to T rows and quant_pack_max_pack() blocks per unit.
    const int lpr = D / 8;
    const int T = (256 / lpr) * 8;
    int tl = 0;
    while ((1 << tl) < T) ++tl;
    a.chunk_rows = T;
    a.rows_log2 = tl;
    const int max_pack = varq::quant_pack_max_pack();
    int units = 0, max_nc = 1, pack_rows = 0, pack_blocks = 0;
    bool in_pack = false;
    for (int g = 0; g < G_in; ++g) {
        a.off[g] = group_offsets[g];
        const int n = group_offsets[g + 1] - group_offsets[g];
        if (n > T) {
            const int nc = (n + T - 1) / T;
            a.unit_start[g] = units;
            units += nc;
            max_nc = std::max(max_nc, nc);
            in_pack = false;
        } else if (in_pack && pack_rows + n <= T && pack_blocks < max_pack) {
            a.unit_start[g] = units - 1;
            pack_rows += n;
            ++pack_blocks;
        } else {
            a.unit_start[g] = units++;
            in_pack = true;
            pack_rows = n;
            pack_blocks = 1;
        }
    }
    // the kernel addresses a unit's rows and a (batch, head)'s word planes with
    // 32-bit byte offsets
    if ((int64_t)T * sx_l * 2 >= ((int64_t)1 << 31) || (int64_t)a.W * L_cap * 4 >= ((int64_t)1 << 31))
        return fail(VARQ_EUNSUPPORTED,
                    "quantize_pack: token stride %lld or cache length %lld too large for 32-bit offsets",
                    (long long)sx_l, (long long)L_cap);
    a.off[G_in] = group_offsets[G_in];
    a.unit_start[G_in] = units;
    a.units_per_bh = units;
    a.n_units = (int64_t)B * H * units;
    a.n_units_one = a.n_units;
    *split = max_nc > 1;
    *max_chunks = max_nc;

    // LDS regions (bytes, 16-aligned): block maxima [max_pack][D], scales and
    // reciprocals [max_pack + 2][D], the staging area for words or code rows
    // (words at 4, 7, 8 bits, code rows at 2, 3, 5, 6 bits; the kernel takes
    // the same choice), then the block-offset and unit-start tables.
    {
        auto up16 = [](int64_t v) { return (int)((v + 15) / 16 * 16); };
        const bool direct = bits == 4 || bits == 7 || bits == 8;
        const int64_t stage = direct ? (int64_t)a.W * (T + 1) * 4 : (int64_t)T * (D >= 64 ? D + 4 : D);
        int o = 0;
        a.lds_max = o;   o += up16((int64_t)max_pack * D * 4);
        a.lds_s = o;     o += up16((int64_t)(max_pack + 2) * D * 4);
        a.lds_y = o;     o += up16((int64_t)(max_pack + 2) * D * 4);
        a.lds_codes = o; o += up16(stage);
        a.lds_off = o;   o += up16((int64_t)(G_in + 1) * 4);
        a.lds_us = o;    o += up16((int64_t)(G_in + 1) * 4);
        a.lds_bytes = o;
    }
    return VARQ_OK;
}

// Launches a prepared quantize+pack (one tensor, or two whose units follow
// each other in one non-split launch).
int qp_launch(varq::QuantPackArgs &a, int bits, bool split, int max_nc, void *stream) {
    const int D = a.D;
    int grid = 0;
    if (split) {
        const int resident = varq::quant_pack_resident_blocks(bits, a.lds_bytes);
        if (resident <= 0) return fail(VARQ_ELAUNCH, "quantize_pack: cannot query the device occupancy");
        grid = (int)std::min<int64_t>(a.n_units, resident);
        // chunks of one block wait for each other: all work-groups must be
        // resident and no block may have more chunks than there are work-groups
        if (max_nc > grid)
            return fail(VARQ_EUNSUPPORTED, "quantize_pack: a block of %d chunks exceeds the %d resident work-groups",
                        max_nc, grid);
        const size_t bhg = (size_t)(a.x2 ? 2 : 1) * a.B * a.H * a.G;
        uint32_t *sync = nullptr;
        uint64_t *slots = nullptr;
        if (int r = scratch_for(static_cast<hipStream_t>(stream), ((size_t)a.n_units + bhg) * D, &sync, &slots))
            return r;
        a.sync = sync;
        a.part = slots;
        a.fin = slots + (size_t)a.n_units * D;
    } else {
        // whole blocks only: one work-group per unit
        grid = (int)std::min<int64_t>(a.n_units, (int64_t)1 << 30);
    }
    return launch_status(varq::launch_quant_pack(a, bits, grid, split, static_cast<hipStream_t>(stream)),
                         "quantize_pack");
}


}  // namespace

extern "C" {

int varq_codes_per_word(int bits) { return (bits >= 2 && bits <= 8) ? 32 / bits : 0; }

int varq_words_per_row(int head_dim, int bits) {
    if (bits < 2 || bits > 8 || head_dim < 1) return 0;
    return words_per_row(head_dim, bits);
}

int varq_cache_bytes(int B, int H, int head_dim, int64_t L_cap, int64_t G_cap, int bits,
                     int64_t *packed_bytes, int64_t *scale_bytes) {
    if (int r = check_bits(bits)) return r;
    if (B < 1 || H < 1 || head_dim < 1 || L_cap < 0 || G_cap < 0)
        return fail(VARQ_EINVAL, "cache_bytes: sizes must be positive (B=%d H=%d D=%d L_cap=%lld G_cap=%lld)",
                    B, H, head_dim, (long long)L_cap, (long long)G_cap);
    const int64_t W = words_per_row(head_dim, bits);
    if (packed_bytes) *packed_bytes = (int64_t)B * H * W * L_cap * 4;
    if (scale_bytes) *scale_bytes = (int64_t)B * H * G_cap * head_dim * 4;
    return ok();
}

int varq_quantize_pack(const void *x, int64_t sx_b, int64_t sx_l, int64_t sx_h,
                       int B, int H, int D, int64_t L_in,
                       const int32_t *group_offsets, int G_in, int bits,
                       int32_t *packed, int64_t L_cap, int64_t tok_start,
                       float *scales, int64_t G_cap, int64_t group_start,
                       void *stream) {
    varq::QuantPackArgs a;
    bool empty = false, split = false;
    int max_nc = 1;
    if (int r = qp_setup(x, sx_b, sx_l, sx_h, B, H, D, L_in, group_offsets, G_in, bits, packed, L_cap, tok_start,
                         scales, G_cap, group_start, a, &empty, &split, &max_nc))
        return r;
    if (empty) return ok();
    return qp_launch(a, bits, split, max_nc, stream);
}

int varq_quantize_pack_kv(const void *k, int64_t sk_b, int64_t sk_l, int64_t sk_h,
                          const void *v, int64_t sv_b, int64_t sv_l, int64_t sv_h,
                          int B, int H, int D, int64_t L_in,
                          const int32_t *group_offsets, int G_in, int bits,
                          int32_t *packed_k, float *scales_k, int32_t *packed_v, float *scales_v,
                          int64_t L_cap, int64_t tok_start, int64_t G_cap, int64_t group_start,
                          void *stream) {
    varq::QuantPackArgs a, av;
    bool empty = false, split = false;
    int max_nc = 1;
    if (int r = qp_setup(k, sk_b, sk_l, sk_h, B, H, D, L_in, group_offsets, G_in, bits, packed_k, L_cap, tok_start,
                         scales_k, G_cap, group_start, a, &empty, &split, &max_nc))
        return r;
    if (int r = qp_setup(v, sv_b, sv_l, sv_h, B, H, D, L_in, group_offsets, G_in, bits, packed_v, L_cap, tok_start,
                         scales_v, G_cap, group_start, av, &empty, &split, &max_nc))
        return r;
    if (empty) return ok();
    if (packed_k == packed_v || scales_k == scales_v)
        return fail(VARQ_EINVAL, "quantize_pack_kv: K and V need caches of their own");
    a.x2 = av.x;
    a.sx2_b = av.sx_b; a.sx2_l = av.sx_l; a.sx2_h = av.sx_h;
    a.packed2 = av.packed;
    a.scales2 = av.scales;
    a.n_units = 2 * a.n_units_one;
    return qp_launch(a, bits, split, max_nc, stream);
}

int64_t varq_grouped_scale_count(int mode, int B, int64_t L, int H, int D, int G) {
    if (B < 0 || L < 0 || H < 0 || D < 0 || G < 0) return -1;
    switch (mode) {
        case VARQ_GROUP_CHANNEL_BLOCK: return (int64_t)B * H * G * D;
        case VARQ_GROUP_CHANNEL: return (int64_t)B * H * D;
        case VARQ_GROUP_BLOCK: return (int64_t)B * G;
        case VARQ_GROUP_TOKEN_HEAD: return (int64_t)B * H * L;
        case VARQ_GROUP_TOKEN: return (int64_t)B * L;
        case VARQ_GROUP_TENSOR: return 1;
        default: return -1;
    }
}

int varq_quantize_pack_grouped(const void *x, int64_t sx_b, int64_t sx_l, int64_t sx_h,
                               int B, int H, int D, int64_t L,
                               int mode, const int32_t *group_offsets, int G, int bits,
                               int32_t *packed, int64_t L_cap,
                               float *scales, int64_t n_scales, void *stream) {
    if (int r = check_bits(bits)) return r;
    if (mode < VARQ_GROUP_CHANNEL_BLOCK || mode > VARQ_GROUP_TENSOR)
        return fail(VARQ_EINVAL, "quantize_pack_grouped: unknown grouping %d", mode);
    if (B < 1 || H < 1 || L < 1)
        return fail(VARQ_EINVAL, "quantize_pack_grouped: B=%d H=%d L=%lld must be >= 1", B, H, (long long)L);
    if (D < 8 || D > 256 || D % 8 != 0)
        return fail(VARQ_EINVAL, "quantize_pack_grouped: head_dim %d must be a multiple of 8 in 8..256", D);
    if (int r = check_offsets(group_offsets, G, L, "quantize_pack_grouped")) return r;
    const int64_t count = varq_grouped_scale_count(mode, B, L, H, D, G);
    if (n_scales < count)
        return fail(VARQ_ECAPACITY, "quantize_pack_grouped: n_scales=%lld < %lld scales of grouping %d",
                    (long long)n_scales, (long long)count, mode);
    if (mode == VARQ_GROUP_CHANNEL_BLOCK)
        return varq_quantize_pack(x, sx_b, sx_l, sx_h, B, H, D, L, group_offsets, G, bits, packed, L_cap, 0,
                                  scales, G, 0, stream);
    if (mode == VARQ_GROUP_CHANNEL) {
        const int32_t whole[2] = {0, (int32_t)L};
        return varq_quantize_pack(x, sx_b, sx_l, sx_h, B, H, D, L, whole, 1, bits, packed, L_cap, 0,
                                  scales, 1, 0, stream);
    }
    if (!x || !packed || !scales) return fail(VARQ_EINVAL, "quantize_pack_grouped: NULL tensor pointer");
    if (!aligned(x, 16) || sx_b % 8 || sx_l % 8 || sx_h % 8)
        return fail(VARQ_EALIGN, "quantize_pack_grouped: x must be 16-byte aligned with strides that are multiples of 8");
    if (!aligned(packed, 16) || L_cap % 8)
        return fail(VARQ_EALIGN, "quantize_pack_grouped: packed must be 16-byte aligned and L_cap a multiple of 8");
    if (!aligned(scales, 4)) return fail(VARQ_EALIGN, "quantize_pack_grouped: scales must be 4-byte aligned");
    if (L > L_cap)
        return fail(VARQ_ECAPACITY, "quantize_pack_grouped: L=%lld exceeds L_cap=%lld", (long long)L, (long long)L_cap);
    const int W = words_per_row(D, bits);
    const int64_t lim = ((int64_t)1 << 31) - 1;
    if ((int64_t)B * L * H * W > lim || (int64_t)B * L * H * (D / 8) > lim || count > lim)
        return fail(VARQ_EUNSUPPORTED, "quantize_pack_grouped: B*L*H*W or the scale count exceeds 2^31 - 1");

    varq::GroupArgs a;
    std::memset(&a, 0, sizeof(a));
    a.x = static_cast<const uint16_t *>(x);
    a.sx_b = sx_b; a.sx_l = sx_l; a.sx_h = sx_h;
    a.packed = reinterpret_cast<uint32_t *>(packed);
    a.absmax = reinterpret_cast<uint32_t *>(scales);
    a.L_cap = L_cap;
    a.B = B; a.L = (int)L; a.H = H; a.D = D; a.W = W; a.G = G;
    for (int g = 0; g <= G; ++g) a.off[g] = group_offsets[g];
    return launch_status(varq::launch_quant_group(a, mode, bits, count, static_cast<hipStream_t>(stream)),
                         "quantize_pack_grouped");
}

namespace {

int unpack_dequant_impl(const int32_t *packed, const float *scales,
                        int B, int H, int D, int64_t L_cap, int64_t G_cap, int64_t L,
                        const int32_t *group_offsets, int G, int bits,
                        const float *rcos, const float *rsin, void *out, void *stream) {
    if (int r = check_bits(bits)) return r;
    if (B < 1 || H < 1) return fail(VARQ_EINVAL, "unpack_dequant: B=%d H=%d must be >= 1", B, H);
    if (D < 8 || D > 256 || D % 8 != 0)
        return fail(VARQ_EINVAL, "unpack_dequant: head_dim %d must be a multiple of 8 in 8..256", D);
    if (L < 0) return fail(VARQ_EINVAL, "unpack_dequant: L=%lld < 0", (long long)L);
    if (L == 0 && G == 0) return ok();
    if (int r = check_offsets(group_offsets, G, L, "unpack_dequant")) return r;
    if (!packed || !scales || !out) return fail(VARQ_EINVAL, "unpack_dequant: NULL tensor pointer");
    if (!aligned(packed, 16) || L_cap % 8)
        return fail(VARQ_EALIGN, "unpack_dequant: packed must be 16-byte aligned and L_cap a multiple of 8");
    if (!aligned(out, 16)) return fail(VARQ_EALIGN, "unpack_dequant: out must be 16-byte aligned");
    if (!aligned(scales, 4)) return fail(VARQ_EALIGN, "unpack_dequant: scales must be 4-byte aligned");
    if (L > L_cap || G > G_cap)
        return fail(VARQ_ECAPACITY, "unpack_dequant: L=%lld / G=%d exceed L_cap=%lld / G_cap=%lld",
                    (long long)L, G, (long long)L_cap, (long long)G_cap);
    const int64_t items = (int64_t)B * H * L * (D / 8);
    if (items / 256 >= (1LL << 31)) return fail(VARQ_EINVAL, "unpack_dequant: tensor too large");
    if (rcos && (!aligned(rcos, 4) || !aligned(rsin, 4)))
        return fail(VARQ_EALIGN, "unpack_dequant_rope: rope tables must be 4-byte aligned");

    varq::UnpackArgs a;
    std::memset(&a, 0, sizeof(a));
    a.packed = reinterpret_cast<const uint32_t *>(packed);
    a.scales = scales;
    a.out = static_cast<uint16_t *>(out);
    a.rcos = rcos; a.rsin = rsin;
    a.L_cap = L_cap; a.G_cap = G_cap; a.L = L;
    a.B = B; a.H = H; a.D = D; a.W = words_per_row(D, bits); a.G = G;
    for (int g = 0; g <= G; ++g) a.off[g] = group_offsets[g];
    return launch_status(varq::launch_unpack_dequant(a, bits, static_cast<hipStream_t>(stream)), "unpack_dequant");
}

}  // namespace

int varq_unpack_dequant(const int32_t *packed, const float *scales,
                        int B, int H, int D, int64_t L_cap, int64_t G_cap, int64_t L,
                        const int32_t *group_offsets, int G, int bits,
                        void *out, void *stream) {
    return unpack_dequant_impl(packed, scales, B, H, D, L_cap, G_cap, L, group_offsets, G, bits, nullptr, nullptr,
                               out, stream);
}

int varq_unpack_dequant_rope(const int32_t *packed, const float *scales,
                             int B, int H, int D, int64_t L_cap, int64_t G_cap, int64_t L,
                             const int32_t *group_offsets, int G, int bits,
                             const float *rope_cos, const float *rope_sin,
                             void *out, void *stream) {
    if (!rope_cos || !rope_sin) return fail(VARQ_EINVAL, "unpack_dequant_rope: NULL rope table");
    return unpack_dequant_impl(packed, scales, B, H, D, L_cap, G_cap, L, group_offsets, G, bits, rope_cos, rope_sin,
                               out, stream);
}

namespace {

// Packed attention; rcos/rsin non-null: K was quantized before RoPE and its
// tiles are rotated after dequantization (tables [L_kv, D/2]).
int packed_attention_impl(const void *q, int64_t sq_b, int64_t sq_l, int64_t sq_h,
                          int B, int H, int D, int64_t Lq,
                          const int32_t *packed_k, const float *scales_k,
                          const int32_t *packed_v, const float *scales_v,
                          int64_t L_cap, int64_t G_cap, int64_t L_kv,
                          const int32_t *group_offsets, int G, int bits,
                          float softmax_scale,
                          void *out, int64_t so_b, int64_t so_l, int64_t so_h,
                          const float *rcos, const float *rsin, void *stream) {
    if (int r = check_bits(bits)) return r;
    if (B < 1 || H < 1) return fail(VARQ_EINVAL, "packed_attention: B=%d H=%d must be >= 1", B, H);
    if (D != 64 && D != 128)
        return fail(VARQ_EUNSUPPORTED, "packed_attention: head_dim %d not implemented (64 or 128)", D);
    if (Lq < 0) return fail(VARQ_EINVAL, "packed_attention: Lq=%lld < 0", (long long)Lq);
    if (Lq == 0) return ok();
    if (L_kv < 1) return fail(VARQ_EINVAL, "packed_attention: the window is empty (L_kv=%lld)", (long long)L_kv);
    if (int r = check_offsets(group_offsets, G, L_kv, "packed_attention")) return r;
    if (!q || !packed_k || !scales_k || !packed_v || !scales_v || !out)
        return fail(VARQ_EINVAL, "packed_attention: NULL tensor pointer");
    if (!std::isfinite(softmax_scale) || softmax_scale <= 0.0f)
        return fail(VARQ_EINVAL, "packed_attention: softmax_scale must be finite and > 0");
    if (!aligned(q, 16) || sq_b % 8 || sq_l % 8 || sq_h % 8)
        return fail(VARQ_EALIGN, "packed_attention: q must be 16-byte aligned with strides that are multiples of 8");
    if (!aligned(out, 8) || so_b % 4 || so_l % 4 || so_h % 4)
        return fail(VARQ_EALIGN, "packed_attention: out must be 8-byte aligned with strides that are multiples of 4");
    if (!aligned(packed_k, 16) || !aligned(packed_v, 16) || L_cap % 8)
        return fail(VARQ_EALIGN, "packed_attention: packed caches must be 16-byte aligned and L_cap a multiple of 8");
    if (!aligned(scales_k, 4) || !aligned(scales_v, 4))
        return fail(VARQ_EALIGN, "packed_attention: scales must be 4-byte aligned");
    if (L_kv > L_cap || G > G_cap)
        return fail(VARQ_ECAPACITY, "packed_attention: L_kv=%lld / G=%d exceed L_cap=%lld / G_cap=%lld",
                    (long long)L_kv, G, (long long)L_cap, (long long)G_cap);
    if ((rcos == nullptr) != (rsin == nullptr))
        return fail(VARQ_EINVAL, "packed_attention_rope: rope_cos and rope_sin must both be given");
    if (rcos && (!aligned(rcos, 4) || !aligned(rsin, 4)))
        return fail(VARQ_EALIGN, "packed_attention_rope: rope tables must be 4-byte aligned");
    const int qtile = varq::attention_q_tile();
    const int64_t n_qtiles = (Lq + qtile - 1) / qtile;
    if (n_qtiles * B * H >= (1LL << 31) - 8) return fail(VARQ_EINVAL, "packed_attention: grid too large");

    varq::AttnArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = static_cast<const uint16_t *>(q);
    a.sq_b = sq_b; a.sq_l = sq_l; a.sq_h = sq_h;
    a.pk = reinterpret_cast<const uint32_t *>(packed_k);
    a.pv = reinterpret_cast<const uint32_t *>(packed_v);
    a.sk = scales_k; a.sv = scales_v;
    a.out = static_cast<uint16_t *>(out);
    a.so_b = so_b; a.so_l = so_l; a.so_h = so_h;
    a.L_cap = L_cap; a.G_cap = G_cap; a.L_kv = L_kv; a.Lq = Lq;
    a.B = B; a.H = H; a.W = words_per_row(D, bits); a.G = G;
    a.n_qtiles = (int)n_qtiles;
    a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
    a.rcos = rcos; a.rsin = rsin;
    for (int g = 0; g <= G; ++g) a.off[g] = group_offsets[g];
    // an under-filled grid runs its KV tiles in ranges, merged afterwards
    if (int r = setup_kv_ranges(a, D, stream)) return r;
    return launch_status(varq::launch_packed_attention(a, D, bits, static_cast<hipStream_t>(stream)),
                         "packed_attention");
}

}  // namespace

int varq_packed_attention(const void *q, int64_t sq_b, int64_t sq_l, int64_t sq_h,
                          int B, int H, int D, int64_t Lq,
                          const int32_t *packed_k, const float *scales_k,
                          const int32_t *packed_v, const float *scales_v,
                          int64_t L_cap, int64_t G_cap, int64_t L_kv,
                          const int32_t *group_offsets, int G, int bits,
                          float softmax_scale,
                          void *out, int64_t so_b, int64_t so_l, int64_t so_h,
                          void *stream) {
    return packed_attention_impl(q, sq_b, sq_l, sq_h, B, H, D, Lq, packed_k, scales_k, packed_v, scales_v,
                                 L_cap, G_cap, L_kv, group_offsets, G, bits, softmax_scale, out, so_b, so_l, so_h,
                                 nullptr, nullptr, stream);
}

int varq_packed_attention_rope(const void *q, int64_t sq_b, int64_t sq_l, int64_t sq_h,
                               int B, int H, int D, int64_t Lq,
                               const int32_t *packed_k, const float *scales_k,
                               const int32_t *packed_v, const float *scales_v,
                               int64_t L_cap, int64_t G_cap, int64_t L_kv,
                               const int32_t *group_offsets, int G, int bits,
                               float softmax_scale,
                               void *out, int64_t so_b, int64_t so_l, int64_t so_h,
                               const float *rope_cos, const float *rope_sin, void *stream) {
    if (!rope_cos || !rope_sin) return fail(VARQ_EINVAL, "packed_attention_rope: NULL rope table");
    return packed_attention_impl(q, sq_b, sq_l, sq_h, B, H, D, Lq, packed_k, scales_k, packed_v, scales_v,
                                 L_cap, G_cap, L_kv, group_offsets, G, bits, softmax_scale, out, so_b, so_l, so_h,
                                 rope_cos, rope_sin, stream);
}

int varq_bf16_attention(const void *q, int64_t sq_b, int64_t sq_l, int64_t sq_h,
                        int B, int H, int D, int64_t Lq,
                        const void *k, const void *v, int64_t L_rows, int64_t L_kv,
                        float softmax_scale,
                        void *out, int64_t so_b, int64_t so_l, int64_t so_h,
                        void *stream) {
    if (B < 1 || H < 1) return fail(VARQ_EINVAL, "bf16_attention: B=%d H=%d must be >= 1", B, H);
    if (D != 64 && D != 128)
        return fail(VARQ_EUNSUPPORTED, "bf16_attention: head_dim %d not implemented (64 or 128)", D);
    if (Lq < 0) return fail(VARQ_EINVAL, "bf16_attention: Lq=%lld < 0", (long long)Lq);
    if (Lq == 0) return ok();
    if (L_kv < 1) return fail(VARQ_EINVAL, "bf16_attention: the window is empty (L_kv=%lld)", (long long)L_kv);
    if (L_kv > L_rows)
        return fail(VARQ_ECAPACITY, "bf16_attention: L_kv=%lld exceeds the %lld rows of k and v",
                    (long long)L_kv, (long long)L_rows);
    if (!q || !k || !v || !out) return fail(VARQ_EINVAL, "bf16_attention: NULL tensor pointer");
    if (!std::isfinite(softmax_scale) || softmax_scale <= 0.0f)
        return fail(VARQ_EINVAL, "bf16_attention: softmax_scale must be finite and > 0");
    if (!aligned(q, 16) || sq_b % 8 || sq_l % 8 || sq_h % 8)
        return fail(VARQ_EALIGN, "bf16_attention: q must be 16-byte aligned with strides that are multiples of 8");
    if (!aligned(out, 8) || so_b % 4 || so_l % 4 || so_h % 4)
        return fail(VARQ_EALIGN, "bf16_attention: out must be 8-byte aligned with strides that are multiples of 4");
    if (!aligned(k, 16) || !aligned(v, 16))
        return fail(VARQ_EALIGN, "bf16_attention: k and v must be 16-byte aligned");
    const int qtile = varq::attention_q_tile();
    const int64_t n_qtiles = (Lq + qtile - 1) / qtile;
    if (n_qtiles * B * H >= (1LL << 31) - 8) return fail(VARQ_EINVAL, "bf16_attention: grid too large");

    varq::AttnArgs a;
    std::memset(&a, 0, sizeof(a));
    a.q = static_cast<const uint16_t *>(q);
    a.sq_b = sq_b; a.sq_l = sq_l; a.sq_h = sq_h;
    a.kd = static_cast<const uint16_t *>(k);
    a.vd = static_cast<const uint16_t *>(v);
    a.out = static_cast<uint16_t *>(out);
    a.so_b = so_b; a.so_l = so_l; a.so_h = so_h;
    a.L_cap = L_rows; a.G_cap = 1; a.L_kv = L_kv; a.Lq = Lq;
    a.B = B; a.H = H; a.W = D / 8; a.G = 1;
    a.n_qtiles = (int)n_qtiles;
    a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
    a.off[0] = 0;
    a.off[1] = (int32_t)L_kv;
    if (int r = setup_kv_ranges(a, D, stream)) return r;
    return launch_status(varq::launch_dense_attention(a, D, static_cast<hipStream_t>(stream)), "bf16_attention");
}

int varq_quantize_pack_check(void *stream) {
    const hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(VARQ_ELAUNCH, "quantize_pack_check: no current device");
    uint32_t *sync = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        auto it = g_scratch.find({dev, st});
        if (it != g_scratch.end()) sync = it->second.sync;
    }
    if (!sync) return VARQ_OK;   // no cooperative launch on this stream yet
    uint32_t status = 0;
    if (hipStreamSynchronize(st) != hipSuccess ||
        hipMemcpy(&status, sync + 2, sizeof(status), hipMemcpyDeviceToHost) != hipSuccess)
        return fail(VARQ_ELAUNCH, "quantize_pack_check: cannot read the exchange status");
    if (status == 0) return VARQ_OK;
    if (hipMemset(sync + 2, 0, sizeof(status)) != hipSuccess)
        return fail(VARQ_ELAUNCH, "quantize_pack_check: cannot clear the exchange status");
    return fail(VARQ_ELAUNCH, "quantize_pack: a cross-work-group wait on this stream hit its time bound; "
                              "outputs of the calls since the last check are not valid");
}

const char *varq_last_error(void) { return g_last_error.c_str(); }

const char *varq_version(void) { return "varq-mi355x 0.1 (gfx950)"; }

}  // extern "C"
