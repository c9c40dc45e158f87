// Index maps of the tiled GEMM kernels: tile order, LDS staging layout,
// fragment reads and accumulator ownership.  Pure integer functions, used by
// the kernels and compiled on the host by the property checks.
#pragma once

#if defined(__HIPCC__)
#define TG_HD __host__ __device__ __forceinline__
#else
#define TG_HD inline
#endif

namespace tg {

constexpr int kXcdCount = 8;    // XCDs per MI355X; workgroups go to them round-robin
constexpr int kRowBytes = 128;  // bytes of K staged per operand row per stage
constexpr int kChunkBytes = 16; // one vector copy per lane (8 x 16-bit or 4 x fp32)
constexpr int kChunksPerRow = kRowBytes / kChunkBytes;

// ---------------------------------------------------------------- tile order
//
// Workgroup `wg` of `nwg` -> output tile (tm, tn).  XCD x (= wg % 8) receives a
// contiguous range of logical tile ids; logical ids then walk the tiles in
// groups of `group_m` tile-rows, down the rows of a group before moving one
// tile-column right, so the tiles resident on one XCD at a time form a compact
// block that shares A and B slabs in that XCD's L2 (cuTile.jl tutorial
// "Matrix Multiplication", "Where to go from here": grouped traversal).
struct TileCoord {
    int tm, tn;
};

// Position of workgroup wg of nwg (dispatched round-robin over the XCDs) in
// an order where the workgroups of one XCD are consecutive.
TG_HD int xcd_order(int wg, int nwg) {
    const int xcd = wg % kXcdCount, slot = wg / kXcdCount;
    const int base = nwg / kXcdCount, rem = nwg % kXcdCount;
    return (xcd < rem) ? xcd * (base + 1) + slot : rem * (base + 1) + (xcd - rem) * base + slot;
}

// Tile t of the grouped walk: group_m tile-rows at a time, column by column.
TG_HD TileCoord grouped_tile(int t, int tiles_m, int tiles_n, int group_m) {
    const int per_group = group_m * tiles_n;
    const int g = t / per_group;
    const int first_m = g * group_m;
    const int gm = (tiles_m - first_m < group_m) ? tiles_m - first_m : group_m;
    const int within = t - g * per_group;
    TileCoord c;
    c.tm = first_m + within % gm;
    c.tn = within / gm;
    return c;
}

TG_HD TileCoord tile_of(int wg, int nwg, int tiles_m, int tiles_n, int group_m) {
    return grouped_tile(xcd_order(wg, nwg), tiles_m, tiles_n, group_m);
}

// ---------------------------------------------------------------- LDS layout
//
// One operand's part of a stage is `rows` rows of 128 bytes.  Logical 16-byte
// chunk c of row r sits in slot c ^ lds_swizzle(r).  For any 8 consecutive rows
// the swizzle takes 8 distinct values, and for any 16 consecutive rows of one
// parity it takes 8 distinct values, so a fixed logical chunk read or written
// by 8 (or 16) lanes on consecutive rows lands in distinct 16-byte slots
// modulo 128 (or 256) bytes.
TG_HD int lds_swizzle(int row) { return (row & 7) ^ ((row >> 3) & 1); }

TG_HD int lds_chunk_offset(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ lds_swizzle(row)) * kChunkBytes);
}

// Staging copy: thread t of the 256-thread workgroup copies logical chunk
// stage_chunk(t) of rows stage_row(t, i), i = 0, 1, ..., so eight consecutive
// threads read one contiguous 128-byte row segment from global memory.
TG_HD int stage_chunk(int t) { return t & 7; }
TG_HD int stage_row(int t, int i) { return (t >> 3) + 32 * i; }

// LDS-DMA into 128-byte rows: one instruction moves 64 lanes x 16 bytes into
// 1 KiB of LDS, lane t at byte 16*t of block j, i.e. row 8*j + t/8, physical
// slot t%8.  The lane fetches the logical chunk the swizzle puts in that slot,
// so each group of 8 lanes reads one whole 128-byte row segment.
TG_HD int dma128_row(int j, int lane) { return 8 * j + (lane >> 3); }
TG_HD int dma128_chunk(int j, int lane) { return (lane & 7) ^ lds_swizzle(dma128_row(j, lane)); }

// ---------------------------------------------------------------- 64-byte rows
//
// The streaming (LDS-DMA) kernels stage 64 bytes of K per row per stage;
// chunk c of row r sits in slot c ^ lds64_swizzle(r).  The swizzle was chosen
// by measurement on gfx950 (the SQ_LDS_BANK_CONFLICT counter over the exact
// fragment-read pattern of these kernels): (r >> 2) & 3 reads conflict-free,
// while for example ((r >> 1) ^ (r >> 3)) & 3, which a plain 64-bank model
// predicts conflict-free, costs a 2-way conflict.
constexpr int kRow64Bytes = 64;
constexpr int kChunksPerRow64 = kRow64Bytes / kChunkBytes;

TG_HD int lds64_swizzle(int row) { return (row >> 2) & 3; }

TG_HD int lds64_chunk_offset(int row, int chunk) {
    return row * kRow64Bytes + ((chunk ^ lds64_swizzle(row)) * kChunkBytes);
}

// One LDS-DMA instruction moves 64 lanes x 16 bytes into 1 KiB of LDS: lane t
// lands at byte 16*t of block j, i.e. row 16*j + t/4, physical slot t%4.  The
// lane therefore fetches the logical chunk that the swizzle puts in that slot.
TG_HD int dma_row(int j, int lane) { return 16 * j + (lane >> 2); }
TG_HD int dma_chunk(int j, int lane) { return (lane & 3) ^ lds64_swizzle(dma_row(j, lane)); }

// ---------------------------------------------------------------- MFMA maps
//
// 32x32 MFMA block, operand side: lane l supplies row frag_row(l) of the
// block and logical chunk frag_chunk(l, q) of slab q (each slab is two chunks,
// one per half-wave).  Both operands use the same map, so every product pairs
// equal k.
TG_HD int frag_row(int lane) { return lane & 31; }
TG_HD int frag_chunk(int lane, int q) { return 2 * q + (lane >> 5); }

// 16x16x32 MFMA block: lane l supplies row frag16_row(l) of the block and
// the 8 consecutive k of its k-group frag16_chunk(l) (0..3, one 16-byte chunk
// of a 64-byte K slice; which chunk is the caller's choice, the same on both
// sides); register r of lane l holds output element (acc16_row(l, r),
// acc16_col(l)) of the 16x16 block (rows n, columns m).
TG_HD int frag16_row(int lane) { return lane & 15; }
TG_HD int frag16_chunk(int lane) { return lane >> 4; }
TG_HD int acc16_row(int lane, int r) { return 4 * (lane >> 4) + r; }
TG_HD int acc16_col(int lane) { return lane & 15; }

// Output side: accumulator register r (0..15) of lane l holds element
// (row acc_row(l, r), column acc_col(l)) of the 32x32 block.  Rows of the MFMA
// output are n (B columns), columns are m (A rows).
TG_HD int acc_row(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
TG_HD int acc_col(int lane) { return lane & 31; }

}  // namespace tg
