// Packed weight layout shared by the host packer (qpack.cpp) and the
// launcher (kernels.hip).  Internal to the library: callers only see
// qpack_*_size() and an opaque buffer.
//
// A 16-byte "unit" is what one lane loads with one 16-byte global load:
//   Q8G64: 16 consecutive int8 codes of one row, stored biased as q+128
//          (4 units make one 64-wide group, which has one fp16 scale)
//   Q4G32: the 32 codes of one 32-wide group of one row, nibbles reordered
//          so that each 16-bit half of a dword pairs with one bf16 pair of x
// A row has U = K/16 (Q8) or K/32 (Q4) units.  G lanes share a row (G is a
// power of two dividing U), so one 64-lane load covers 64/G rows.  A tile is
// R such row slots, TR = R*64/G rows, walked in J = U/G steps.  In step j,
// lane l = rho*G + g holds unit j*G + g of row tile*TR + r*(64/G) + rho.
//
// Buffer = [code blocks][meta blocks], both in (tile, step) order:
//   code block (tile, step, r): 1024 bytes, lane l's unit at l*16
//   meta block (tile, step):
//     Q8: for each (rho, group-in-step a = g/4): R fp16 scales (one per r),
//         so the 4 lanes of a group read the same 2R bytes
//     Q4: for each lane l: R dwords (scale | min << 16), one per r
// Rows past N in the last tile are padding: zero scale and min, code bytes
// that decode to zero.  Every weight byte is stored exactly once; the
// padding is at most TR-1 rows.
#pragma once
#include <stdint.h>

namespace qg {

enum { FMT_Q8G64 = 0, FMT_Q4G32 = 1 };

struct Layout {
    int fmt;
    int64_t N, K;
    int group;          // 64 or 32 codes
    int unit_codes;     // 16 or 32 codes per 16-byte unit
    int64_t U;          // units per row
    int G;              // lanes per row (power of two, divides U)
    int R;              // row slots per lane
    int64_t J;          // steps per tile (U / G)
    int TR;             // rows per tile
    int64_t tiles;
    int64_t meta_step_bytes;
    int64_t code_bytes;
    int64_t meta_bytes;
    int64_t total_bytes;  // code + meta, rounded up to 256
};

static const int kRowSlots = 2;

// Chooses G and R for a matrix and fills the byte counts.  Returns false for
// shapes the format cannot hold (K not a whole number of groups, N or K < 1,
// sizes whose offsets would not fit in 63 bits).
static inline bool make_layout(int fmt, int64_t N, int64_t K, Layout* L)
{
    if (fmt != FMT_Q8G64 && fmt != FMT_Q4G32) return false;
    const int group = fmt == FMT_Q8G64 ? 64 : 32;
    if (N < 1 || K < 1 || K % group != 0) return false;
    if (N > (int64_t(1) << 31) - 1 || K > (int64_t(1) << 31) - 1) return false;
    Layout l;
    l.fmt = fmt;
    l.N = N;
    l.K = K;
    l.group = group;
    l.unit_codes = fmt == FMT_Q8G64 ? 16 : 32;
    l.U = K / l.unit_codes;
    int G = 64;
    while (G > 1 && l.U % G != 0) G /= 2;
    // Keep at least two steps per lane when the row allows it, so a tile's
    // cross-lane reduction is spread over more than one unit per lane.
    const int g_min = fmt == FMT_Q8G64 ? 4 : 1;
    while (G > g_min && l.U / G < 2) G /= 2;
    l.G = G;
    l.R = kRowSlots;
    l.J = l.U / G;
    l.TR = l.R * (64 / G);
    l.tiles = (N + l.TR - 1) / l.TR;
    l.meta_step_bytes = fmt == FMT_Q8G64 ? int64_t(32) * l.R : int64_t(256) * l.R;
    l.code_bytes = l.tiles * l.J * l.R * 1024;
    l.meta_bytes = l.tiles * l.J * l.meta_step_bytes;
    l.total_bytes = (l.code_bytes + l.meta_bytes + 255) / 256 * 256;
    *L = l;
    return true;
}

}  // namespace qg
