// Packed weight layout shared by the host packer (qpack.cpp) and the
// launcher (launch.hip, kernel_body.h).  Internal to the library: callers only see
// qpack_*_size() and an opaque buffer.
//
// A 16-byte "unit" is what one lane loads with one 16-byte global load:
//   Q8G64, Q8G128, Q8PC: 16 consecutive signed int8 codes of one row, as
//          they are (4 units make a 64-wide group, 8 a 128-wide group)
//   Q4G32: the 32 codes of one 32-wide group of one row, nibbles reordered
//          so that each 16-bit half of a dword pairs with one bf16 pair of x
//          (dword d holds k = 8d .. 8d + 7: k = 8d + 2p in bits 4p .. 4p + 3,
//          k = 8d + 2p + 1 in bits 16 + 4p .. 19 + 4p)
// A row has U = K/16 (8-bit codes) or K/32 (Q4) units.  G lanes share a row
// (G is a power of two dividing U, at least the units per scale group), so
// one 64-lane load covers 64/G rows.  A tile is R such row slots,
// TR = R*64/G rows, walked in J = U/G steps.  In step j, lane l = rho*G + g
// holds unit j*G + g of row tile*TR + r*(64/G) + rho.
//
// Buffer = [code blocks][meta], both in (tile, step) order:
//   code block (tile, step, r): 1024 bytes, lane l's unit at l*16
//   meta of (tile, step) at code_bytes + tile*(J*meta_step + meta_tile)
//                           + step*meta_step:
//     Q8G64:  for each (rho, group-in-step a = g/4): R fp16 scales (one per
//             r), so the 4 lanes of a group read the same 2R bytes
//     Q8G128: the same with a = g/8 (8 lanes per group)
//     Q4G32:  for each lane l: R dwords (scale | min << 16), one per r
//     Q8PC:   no per-step meta; after a tile's steps, its TR fp32 row scales
//             ordered [rho][r], so lane l's R scales are contiguous
// Rows past N in the last tile are padding: zero codes, scales and mins.  Every weight byte is stored exactly once; the
// padding is at most TR-1 rows.
#pragma once
#include <stdint.h>

namespace qg {

enum { FMT_Q8G64 = 0, FMT_Q4G32 = 1, FMT_Q8G128 = 2, FMT_Q8PC = 3 };

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
    int64_t meta_tile_bytes;  // Q8PC row scales per tile
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
    int group, unit_codes, g_min;
    switch (fmt) {
    case FMT_Q8G64: group = 64; unit_codes = 16; g_min = 4; break;
    case FMT_Q4G32: group = 32; unit_codes = 32; g_min = 1; break;
    case FMT_Q8G128: group = 128; unit_codes = 16; g_min = 8; break;
    case FMT_Q8PC: group = 16; unit_codes = 16; g_min = 1; break;   // K granularity only
    default: return false;
    }
    if (N < 1 || K < 1 || K % group != 0) return false;
    if (N > (int64_t(1) << 31) - 1 || K > (int64_t(1) << 31) - 1) return false;
    Layout l;
    l.fmt = fmt;
    l.N = N;
    l.K = K;
    l.group = group;
    l.unit_codes = unit_codes;
    l.U = K / unit_codes;
    int G = 64;
    while (G > 1 && l.U % G != 0) G /= 2;
    // Keep at least two steps per lane when the row allows it, so a tile's
    // cross-lane reduction is spread over more than one unit per lane.
    while (G > g_min && l.U / G < 2) G /= 2;
    l.G = G;
    l.R = kRowSlots;
    l.J = l.U / G;
    l.TR = l.R * (64 / G);
    l.tiles = (N + l.TR - 1) / l.TR;
    switch (fmt) {
    case FMT_Q8G64: l.meta_step_bytes = int64_t(32) * l.R; l.meta_tile_bytes = 0; break;
    case FMT_Q8G128: l.meta_step_bytes = int64_t(16) * l.R; l.meta_tile_bytes = 0; break;
    case FMT_Q4G32: l.meta_step_bytes = int64_t(256) * l.R; l.meta_tile_bytes = 0; break;
    default: l.meta_step_bytes = 0; l.meta_tile_bytes = int64_t(4) * l.TR; break;
    }
    l.code_bytes = l.tiles * l.J * l.R * 1024;
    l.meta_bytes = l.tiles * (l.J * l.meta_step_bytes + l.meta_tile_bytes);
    l.total_bytes = (l.code_bytes + l.meta_bytes + 255) / 256 * 256;
    *L = l;
    return true;
}

// Gate/up pair layout (Q4G32 only), for a fused SwiGLU epilogue: the packed
// matrix is an ordinary Q4G32 layout of Nv = 2 * ceil(N / RPS) * RPS rows
// (RPS = 64 / G rows per row slot) in which tile t holds gate rows
// t*RPS .. t*RPS + RPS - 1 in row slot 0 and the up rows with the same
// indices in row slot 1, so one lane group ends a tile with both halves of
// each output.  Rows past N are zero padding.  G depends on K alone, so the
// N-row and Nv-row layouts share it.
static_assert(kRowSlots == 2, "gate/up pairs occupy the two row slots of a tile");

static inline bool make_gate_up_layout(int64_t N, int64_t K, Layout* L, int64_t* rows_per_slot)
{
    Layout l0;
    if (!make_layout(FMT_Q4G32, N, K, &l0)) return false;
    const int64_t rps = 64 / l0.G;
    const int64_t Nv = 2 * ((N + rps - 1) / rps) * rps;
    if (!make_layout(FMT_Q4G32, Nv, K, L) || L->G != l0.G) return false;
    *rows_per_slot = rps;
    return true;
}

// Matrix-core ("mma") layout of the 8-bit formats, for the kernel that
// feeds the 16x16x32 bf16 MFMA (m = 2..16 activation rows share the B-side
// weights).  A tile is 16 rows; a step covers 64 consecutive K.  Item
// (tile t, step j) is one 1 KiB block at (t*J + j)*1024 in which lane l
// holds the 16 signed codes of row t*16 + (l mod 16) at
// k = 64j + 16*(l div 16) .. +15: the MFMA's B operand (lane l supplies
// column l mod 16, k-slice l div 16) with no shuffling.  Meta after all
// code blocks:
//   Q8G64:  [tile][64-group][16 rows] fp16 scales
//   Q8G128: [tile][128-group][16 rows] fp16 scales
//   Q8PC:   [tile][16 rows] fp32 row scales
// K must be a multiple of 64 (128 for Q8G128).  Rows past N are padding
// (code 0, scale 0).  Every weight byte is stored once.
//
// Q4G32 uses the same tiles with 128-wide steps, so that an item is still
// 1 KiB: lane l holds four dwords, dword g being the eight codes of row
// t*16 + (l mod 16) at k = 128j + 32g + 8*(l div 16) + e (e = 0..7) as
// their four canonical bytes (e = 2b in the low nibble of byte b, 2b + 1 in
// the high nibble): the B operand of one MFMA (in k order once widened),
// which thus covers exactly one 32-group.  Meta after all code
// blocks: [tile][step][16 rows][4 groups] dwords, scale (fp16) in the low
// half and min (fp16) in the high half.  K must be a multiple of 128.
// Rows past N are padding (code 0, scale 0, min 0).
struct MmaLayout {
    int fmt;
    int64_t N, K;
    int group;              // codes per scale (K for Q8PC)
    int64_t J;              // steps per row (64 wide; 128 for Q4G32)
    int64_t groups;         // scale groups per row
    int64_t tiles;          // 16-row tiles
    int64_t code_bytes;
    int64_t meta_tile_bytes;
    int64_t total_bytes;    // rounded up to 256
};

static const int kMmaRows = 16;

static inline bool make_mma_layout(int fmt, int64_t N, int64_t K, MmaLayout* L)
{
    int group;
    switch (fmt) {
    case FMT_Q8G64: group = 64; break;
    case FMT_Q8G128: group = 128; break;
    case FMT_Q8PC: group = 0; break;
    case FMT_Q4G32: group = 32; break;
    default: return false;
    }
    const int64_t step = fmt == FMT_Q4G32 ? 128 : 64;
    if (N < 1 || K < step || K % step != 0 || (group && K % group != 0)) return false;
    if (N > (int64_t(1) << 31) - 1 || K > (int64_t(1) << 31) - 1) return false;
    MmaLayout l;
    l.fmt = fmt;
    l.N = N;
    l.K = K;
    l.group = group ? group : int(K);
    l.J = K / step;
    l.groups = group ? K / group : 1;
    l.tiles = (N + kMmaRows - 1) / kMmaRows;
    l.code_bytes = l.tiles * l.J * 1024;
    l.meta_tile_bytes = fmt == FMT_Q8PC ? 4 * kMmaRows
                      : fmt == FMT_Q4G32 ? 4 * kMmaRows * l.groups
                                         : 2 * kMmaRows * l.groups;
    l.total_bytes = (l.code_bytes + l.tiles * l.meta_tile_bytes + 255) / 256 * 256;
    *L = l;
    return true;
}

}  // namespace qg
