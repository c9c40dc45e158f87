// Host-side property checks of the kernels' index maps (csrc/tile_math.h),
// compiled with g++ by tests/test_host_maps.py.  Prints one line per failed
// property and exits nonzero if any failed.
//
//  * tile order: a bijection from workgroup ids onto the tile grid;
//  * staging copy: every (row, chunk) of an operand stage written exactly once
//    (the unique-destination rule of the Tylo.jl manual, "Walk through GEMM",
//    section 3), and conflict-free 16-byte LDS writes;
//  * fragment reads: conflict-free (128-byte rows, under a 16-lane / 64-bank
//    and an 8-lane / 32-bank model, both consistent with the counter on
//    gfx950), and both operands cover the same k set;
//  * accumulator ownership: a bijection onto the 32x32 block and, over lanes,
//    waves and blocks, onto the workgroup tile, with acc/lane * threads equal
//    to the tile size (section 1 of the same page: register counts follow from
//    the ownership of the atom and its repetitions).
#include <cstdio>
#include <set>
#include <vector>

#include "tile_math.h"

using namespace tg;

static int failures = 0;
#define CHECK(cond, ...)                  \
    do {                                  \
        if (!(cond)) {                    \
            ++failures;                   \
            std::printf("FAIL: " __VA_ARGS__); \
            std::printf("\n");            \
        }                                 \
    } while (0)

static void check_tile_order() {
    const int shapes[][2] = {{1, 1}, {1, 7}, {3, 1}, {4, 4}, {5, 3}, {32, 32}, {49, 20},
                             {8, 8}, {7, 9}, {17, 13}, {2, 128}, {130, 3}, {97, 41}};
    for (auto& sh : shapes) {
        for (int gm : {1, 2, 4, 8}) {
            const int tm_ = sh[0], tn_ = sh[1], n = tm_ * tn_;
            std::vector<int> seen(n, 0);
            bool in_range = true;
            for (int wg = 0; wg < n; ++wg) {
                TileCoord c = tile_of(wg, n, tm_, tn_, gm);
                if (c.tm < 0 || c.tm >= tm_ || c.tn < 0 || c.tn >= tn_) { in_range = false; continue; }
                seen[c.tm * tn_ + c.tn]++;
            }
            bool bij = in_range;
            for (int v : seen) bij = bij && v == 1;
            CHECK(bij, "tile_of not a bijection for tiles %dx%d group %d", tm_, tn_, gm);
        }
    }
    // 32 consecutive logical tiles of one XCD form a group_m x (32/group_m) block
    const int tm_ = 32, tn_ = 32, n = tm_ * tn_;
    for (int x = 0; x < kXcdCount; ++x) {
        std::set<int> rows, cols;
        for (int slot = 0; slot < 32; ++slot) {
            TileCoord c = tile_of(x + kXcdCount * slot, n, tm_, tn_, 4);
            rows.insert(c.tm);
            cols.insert(c.tn);
        }
        CHECK(rows.size() == 4 && cols.size() == 8, "XCD %d first 32 tiles span %zu rows x %zu cols", x,
              rows.size(), cols.size());
    }
}

// distinct 16-byte slots among `lanes` byte offsets taken `group` at a time,
// modulo `window` bytes
static bool conflict_free(const std::vector<int>& off, int group, int window) {
    for (size_t g0 = 0; g0 + group <= off.size(); g0 += group) {
        std::set<int> slots;
        for (int i = 0; i < group; ++i) slots.insert((off[g0 + i] % window) / kChunkBytes);
        if ((int)slots.size() != group) return false;
    }
    return true;
}

static void check_staging(int rows) {
    std::vector<int> count(rows * kChunksPerRow, 0);
    std::set<int> offsets;
    const int reps = rows / 32;
    for (int t = 0; t < 256; ++t)
        for (int i = 0; i < reps; ++i) {
            const int r = stage_row(t, i), c = stage_chunk(t);
            CHECK(r < rows && c < kChunksPerRow, "staging out of range");
            count[r * kChunksPerRow + c]++;
            offsets.insert(lds_chunk_offset(r, c));
        }
    bool once = true;
    for (int v : count) once = once && v == 1;
    CHECK(once, "staging does not cover %d rows x 8 chunks exactly once", rows);
    CHECK((int)offsets.size() == rows * kChunksPerRow, "LDS destinations not unique (%d rows)", rows);
    for (int o : offsets) CHECK(o >= 0 && o < rows * kRowBytes && o % kChunkBytes == 0, "bad LDS offset %d", o);
    // one ds_write_b128 instruction: 64 lanes of one wave, same i
    for (int w = 0; w < 4; ++w)
        for (int i = 0; i < reps; ++i) {
            std::vector<int> off;
            for (int l = 0; l < 64; ++l) {
                const int t = 64 * w + l;
                off.push_back(lds_chunk_offset(stage_row(t, i), stage_chunk(t)));
            }
            CHECK(conflict_free(off, 8, 128) && conflict_free(off, 16, 256),
                  "staging write conflicts (wave %d rep %d)", w, i);
        }
}

static void check_fragments() {
    for (int q = 0; q < 4; ++q)
        for (int blk = 0; blk < 8; ++blk) {
            std::vector<int> off;
            std::set<int> rowchunks;
            for (int l = 0; l < 64; ++l) {
                const int r = 32 * blk + frag_row(l);
                off.push_back(lds_chunk_offset(r, frag_chunk(l, q)));
                rowchunks.insert(frag_row(l) * 64 + frag_chunk(l, q));
            }
            CHECK(conflict_free(off, 8, 128) && conflict_free(off, 16, 256),
                  "fragment read conflicts (slab %d block %d)", q, blk);
            // each of the 32 rows gets both chunks of the slab exactly once
            CHECK(rowchunks.size() == 64, "slab %d does not give each row both chunks", q);
            for (int r = 0; r < 32; ++r)
                CHECK(rowchunks.count(r * 64 + 2 * q) && rowchunks.count(r * 64 + 2 * q + 1),
                      "row %d misses a chunk of slab %d", r, q);
        }
    // the four slabs cover the eight chunks of a row
    std::set<int> chunks;
    for (int q = 0; q < 4; ++q)
        for (int l = 0; l < 64; ++l) chunks.insert(frag_chunk(l, q));
    CHECK(chunks.size() == 8, "slabs do not cover the 128-byte row");
}

static void check_ownership(int BM, int BN) {
    // 32x32 block
    std::set<int> blk;
    for (int l = 0; l < 64; ++l)
        for (int r = 0; r < 16; ++r) {
            const int row = acc_row(l, r), col = acc_col(l);
            CHECK(row >= 0 && row < 32 && col >= 0 && col < 32, "acc out of block");
            blk.insert(row * 32 + col);
        }
    CHECK(blk.size() == 1024, "accumulator ownership is not a bijection onto 32x32");
    // workgroup tile: 2x2 waves of (BM/2)x(BN/2), blocks of 32x32
    const int WTM = BM / 2, WTN = BN / 2;
    std::vector<int> cover(BM * BN, 0);
    int acc_per_lane = 0;
    for (int wave = 0; wave < 4; ++wave) {
        const int wave_m = wave & 1, wave_n = wave >> 1;
        for (int l = 0; l < 64; ++l) {
            int count = 0;
            for (int i = 0; i < WTN / 32; ++i)
                for (int j = 0; j < WTM / 32; ++j)
                    for (int r = 0; r < 16; ++r) {
                        const int m = wave_m * WTM + 32 * j + acc_col(l);
                        const int n = wave_n * WTN + 32 * i + acc_row(l, r);
                        cover[n * BM + m]++;
                        ++count;
                    }
            acc_per_lane = count;
        }
    }
    bool once = true;
    for (int v : cover) once = once && v == 1;
    CHECK(once, "tile %dx%d not owned exactly once", BM, BN);
    CHECK(acc_per_lane * 256 == BM * BN, "acc/lane %d * 256 != %d*%d", acc_per_lane, BM, BN);
}

// 64-byte-row layout of the streaming kernels: every DMA lane lands exactly
// where the swizzled layout puts its logical chunk, each (row, chunk) of a
// stage is written once, and fragment reads of both slabs are conflict-free.
static void check_dma_layout(int rows) {
    const int blocks = rows * kRow64Bytes / 1024;
    std::vector<int> count(rows * kChunksPerRow64, 0);
    for (int j = 0; j < blocks; ++j)
        for (int t = 0; t < 64; ++t) {
            const int r = dma_row(j, t), c = dma_chunk(j, t);
            CHECK(r < rows && c >= 0 && c < kChunksPerRow64, "dma out of range");
            CHECK(lds64_chunk_offset(r, c) == j * 1024 + 16 * t, "dma lane %d of block %d lands elsewhere", t, j);
            count[r * kChunksPerRow64 + c]++;
        }
    bool once = true;
    for (int v : count) once = once && v == 1;
    CHECK(once, "dma does not cover %d rows x 4 chunks exactly once", rows);
    // (bank conflicts of this layout were measured on the GPU, not modelled:
    // a plain 64-bank model mispredicts 64-byte rows)
    for (int q = 0; q < 2; ++q) {
        std::set<int> rowchunks;
        for (int l = 0; l < 64; ++l) rowchunks.insert(frag_row(l) * 4 + frag_chunk(l, q));
        CHECK(rowchunks.size() == 64, "64-byte-row slab %d does not give each row both chunks", q);
    }
}

// 128-byte-row DMA layout of the wide streaming kernel: lane t of block j lands
// where the swizzled layout puts its logical chunk, every (row, chunk) of a
// stage is written once, and each group of 8 lanes reads one whole row segment.
static void check_dma128_layout(int rows) {
    const int blocks = rows * kRowBytes / 1024;
    std::vector<int> count(rows * kChunksPerRow, 0);
    for (int j = 0; j < blocks; ++j)
        for (int t = 0; t < 64; ++t) {
            const int r = dma128_row(j, t), c = dma128_chunk(j, t);
            CHECK(r < rows && c >= 0 && c < kChunksPerRow, "dma128 out of range");
            CHECK(lds_chunk_offset(r, c) == j * 1024 + 16 * t, "dma128 lane %d of block %d lands elsewhere", t, j);
            count[r * kChunksPerRow + c]++;
        }
    bool once = true;
    for (int v : count) once = once && v == 1;
    CHECK(once, "dma128 does not cover %d rows x 8 chunks exactly once", rows);
    for (int j = 0; j < blocks; ++j)
        for (int g = 0; g < 8; ++g) {
            std::set<int> chunks;
            for (int t = 8 * g; t < 8 * g + 8; ++t) {
                CHECK(dma128_row(j, t) == dma128_row(j, 8 * g), "dma128 lane group %d spans rows", g);
                chunks.insert(dma128_chunk(j, t));
            }
            CHECK(chunks.size() == 8, "dma128 lane group %d of block %d misses part of its row", g, j);
        }
}

int main() {
    check_dma128_layout(256);
    check_dma128_layout(128);
    check_tile_order();
    check_dma_layout(256);
    check_dma_layout(128);
    check_staging(128);
    check_staging(256);
    check_fragments();
    check_ownership(128, 128);
    check_ownership(256, 256);
    if (failures) {
        std::printf("%d property failures\n", failures);
        return 1;
    }
    std::printf("all index-map properties hold\n");
    return 0;
}
