// varq_tile_math.h - index arithmetic of the packed-attention tile loads,
// shared by the gfx950 kernel and the host-side self-test that checks it
// stays inside the cache.
#pragma once

#include <hip/hip_runtime.h>

namespace varq {

// Tokens per KV tile of the packed attention, and tokens per load item: one
// item is 4 consecutive tokens of one word plane, a 16-byte load.
constexpr int kAttnTileTokens = 64;
constexpr int kAttnItemTokens = 4;

// First token that item t4 (0..15) of the tile starting at token n0 loads,
// for a window of L_kv >= 1 tokens. Items past the window's last 4-token group
// load that group again (their tokens are masked out of the scores), so a load
// never reaches past round_up(L_kv, 4) - 1 <= L_cap - 1 (the cache capacity
// is a multiple of 8 and at least L_kv), and stays 16-byte aligned.
__host__ __device__ inline int attn_item_first_token(int n0, int t4, int L_kv) {
    const int last = (L_kv - 1) & ~(kAttnItemTokens - 1);
    const int t = n0 + kAttnItemTokens * t4;
    return t < last ? t : last;
}

}  // namespace varq
