// tile_layout.h -- tile shapes, stage/K-tile choices and the LDS layout of a
// pipelined GEMM tile.  Plain constexpr C++ with no HIP dependency: the
// kernels, the host-side configuration code and a host test all include it,
// so the three agree by construction.
//
// Background.  Software pipelining keeps the next K-tile's global->shared
// copy in flight while the current tile is multiplied ("CUDA Kernel Study:
// Pipelining", Background / Case 1 / Case 2).  The shared-memory cost is
// slots x tile, and the tile must stay under the occupancy cliff set by the
// per-block shared-memory budget ("pipeline-gpu-kernel", step 1).  On gfx950
// the budget is the 160 KiB LDS of one CU; these kernels run one workgroup
// per CU, so a workgroup may use all of it.
//
// LDS layout.  Every operand tile is a grid of 16-byte chunks: `rows` rows of
// `cpr` chunks (cpr = chunks per row).  A tile is written row-major in chunk
// order, lane-contiguous (one 16-byte chunk per lane per instruction), which
// is the only order the direct-to-LDS load can produce.  Inside a row the
// chunk a row's logical chunk c lives in is c ^ swz(row): an XOR swizzle that
// costs no LDS bytes (padding would cost 1/cpr of the tile).  gfx950's LDS
// has 64 banks of 4 bytes and serves a 16-byte read in 4 clocks of 16 lanes;
// measured lane pair by lane pair (SQ_LDS_BANK_CONFLICT), lane l goes in
// clock 2 (l / 32) + the parity of bits 2-4 of l, so lanes 0-3, 12-15,
// 20-23 and 24-27 share a clock, and 4-7, 8-11, 16-19 and 28-31 another.
// The 16 lanes of one clock must hit 16 different 16-byte bank groups.  Two
// fragment reads use the tiles: for the 32x32 MFMA blocks lane l fetches row
// (l % 32) at chunk (c0 + l / 32); for the 16x16 blocks row (16 h + l % 16)
// at chunk (c0 + l / 16), c0 a multiple of 4.  The swizzles below are
// conflict-free for both reads under that grouping (and under 16 consecutive
// lanes per clock), and were measured so on the hardware.
// The padding/swizzling remedy for shared-memory bank conflicts is the next
// step the pipelining study names (Detailed Analysis, item 5).
#ifndef PIPEGEMM_TILE_LAYOUT_H
#define PIPEGEMM_TILE_LAYOUT_H

#include <stdint.h>

namespace pg {

enum DType : int { DT_I8 = 0, DT_F16 = 1, DT_BF16 = 2, DT_F32 = 3 };
enum Layout : int { LAYOUT_RR = 0, LAYOUT_RC = 1 };
// VAR_REG_KTAIL is VAR_REG for a K that is not a multiple of 16 bytes: its
// first (ragged) K-tile load reads the partial chunk at K exactly.
enum Variant : int { VAR_REG = 0, VAR_DIRECT = 1, VAR_REG_KTAIL = 2 };
enum TileClass : int { TILE_L = 0, TILE_M = 1, TILE_T = 2, TILE_W = 3, TILE_COUNT = 4 };

constexpr int kMaxStages = 4;

constexpr int kLdsBudget = 160 * 1024;   // bytes of LDS per CU on gfx950
constexpr int kChunk = 16;               // bytes per lane per load

constexpr int in_size(int dt) { return dt == DT_I8 ? 1 : (dt == DT_F32 ? 4 : 2); }
constexpr int out_size(int dt) { return dt == DT_I8 ? 4 : (dt == DT_F32 ? 4 : 2); }
// elements per 16-byte chunk
constexpr int epc(int dt) { return kChunk / in_size(dt); }

// Workgroup tile and wave grid of each class.  Each wave owns a
// (bm/wm) x (bn/wn) block of C made of 32x32 MFMA blocks.  TILE_W is the
// 256x256 tile with 8 waves (2 per SIMD, 128x64 each): while one wave of a
// SIMD waits (on its loads, on the barrier), the other can issue MFMAs.
// wk > 1 splits each K-tile's k-steps over wk waves per C block (wave k
// group g takes the g-th run of steps); after the K loop the groups' partial
// accumulators are added through LDS.  The 32x64 tile runs two k groups:
// its 2 x 1 waves of 32x32 left two of a CU's four SIMDs idle, and with the
// K-tile's steps split over four waves each wave issues half the MFMAs and
// fragment reads and a quarter of the loads (measured: fp32 256^3 7.5 ->
// 5.9 us; the skinny bf16 shape's register-staged pairs 35-38 -> 32 us).
struct TileShape { int bm, bn, wm, wn, wk; };
constexpr TileShape tile_shape(int tc) {
    return tc == TILE_L ? TileShape{256, 256, 2, 2, 1}
         : tc == TILE_W ? TileShape{256, 256, 2, 4, 1}
         : tc == TILE_M ? TileShape{128, 128, 2, 2, 1}
                        : TileShape{32, 64, 1, 2, 2};
}

// The 3-stage direct-to-LDS ring of the 256x256 classes is split by
// operand: three A slots and two B slots of a full-width K-tile, exactly the
// 160 KiB of LDS.  The A tile is loaded two K-tiles ahead and the B tile one
// ahead, where three whole slots would need 192 KiB.
constexpr bool split_ring(int tc, int stages, int variant) {
    return variant == VAR_DIRECT && stages == 3 && (tc == TILE_L || tc == TILE_W);
}

// Chunks per K-contiguous row of a K-tile.  The large tile halves its K-tile
// where the ring would not fit the LDS budget otherwise (the remedy the
// skill gives for a buffer over the cliff: halve BK): at 4 stages, and at 3
// stages for the register-staged variant.
constexpr int cpr_k(int tc, int stages, int variant) {
    return (tc == TILE_L || tc == TILE_W) ? ((stages <= 2 || split_ring(tc, stages, variant)) ? 8 : 4)
         : tc == TILE_M ? 8 : 16;
}
constexpr int block_k(int dt, int tc, int stages, int variant) { return cpr_k(tc, stages, variant) * epc(dt); }

// MFMA block edge: 16x16 blocks (16x16x32 fp16/bf16, 16x16x64 int8) for the
// 4-wave 256x256 tile's 2-3 stage direct rings with full-width K-tiles
// (both layouts); 32x32 blocks for every other instance.  The matrix
// cores hold a higher clock on the 16x16 blocks; both give the same bits.
constexpr bool mfma_block16(int dt, int layout, int tc, int stages, int variant) {
    return tc == TILE_L && variant == VAR_DIRECT && stages >= 2 && cpr_k(tc, stages, variant) >= 8 &&
           (layout == LAYOUT_RC || layout == LAYOUT_RR) && dt != DT_F32;
}

// LDS slots of the ring and register staging sets per variant:
//  direct-to-LDS: `stages` slots, stages-1 tiles in flight, no staging set
//  (split ring: three A slots, two B slots);
//  register-staged: min(stages, 2) slots and max(1, stages-1) staging sets,
//  each holding one tile in flight.
constexpr int lds_slots(int variant, int stages) {
    return variant == VAR_DIRECT ? stages : (stages < 2 ? stages : 2);
}
constexpr int reg_sets(int variant, int stages) {
    return variant == VAR_DIRECT ? 0 : (stages > 1 ? stages - 1 : 1);
}
constexpr int tiles_in_flight(int variant, int stages) {
    return variant == VAR_DIRECT ? stages - 1 : reg_sets(variant, stages);
}

// Bytes of one ring slot (A tile followed by B tile), and of the ring.
constexpr int slot_bytes(int dt, int tc, int stages, int variant) {
    return (tile_shape(tc).bm + tile_shape(tc).bn) * block_k(dt, tc, stages, variant) * in_size(dt);
}
constexpr int ring_bytes(int dt, int tc, int stages, int variant) {
    return split_ring(tc, stages, variant)
               ? (3 * tile_shape(tc).bm + 2 * tile_shape(tc).bn) * block_k(dt, tc, stages, variant) * in_size(dt)
               : slot_bytes(dt, tc, stages, variant) * lds_slots(variant, stages);
}
// The epilogue reuses LDS to stage one 32-row strip of C per wave.  A strip
// row is the wave's block width, plus 16 bytes of padding that spreads the
// rows over the LDS banks for 4-byte outputs; 2-byte outputs are placed by
// strip_off instead (no padding).
constexpr int strip_row_bytes(int dt, int tc) {
    return tile_shape(tc).bn / tile_shape(tc).wn * out_size(dt) + (out_size(dt) == 2 ? 0 : kChunk);
}
constexpr int epilogue_bytes(int dt, int tc) {
    return 32 * strip_row_bytes(dt, tc) * tile_shape(tc).wm * tile_shape(tc).wn;
}
constexpr int threads(int tc) { return tile_shape(tc).wm * tile_shape(tc).wn * tile_shape(tc).wk * 64; }
// LDS for adding the k groups' partial accumulators (wk > 1): the groups
// g >= 1 each store their 32x32-block accumulators (16 words per lane and
// block) for the group-0 waves to add.
constexpr int kred_bytes(int tc) {
    return (tile_shape(tc).wk - 1) * tile_shape(tc).wm * tile_shape(tc).wn *
           (tile_shape(tc).bm / tile_shape(tc).wm / 32) * (tile_shape(tc).bn / tile_shape(tc).wn / 32) * 64 * 64;
}
constexpr int max3(int a, int b, int c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); }
constexpr int lds_bytes(int dt, int tc, int stages, int variant) {
    return max3(ring_bytes(dt, tc, stages, variant), epilogue_bytes(dt, tc), kred_bytes(tc));
}

// 16-byte loads per lane per K-tile for each operand.
constexpr int loads_a(int dt, int tc, int stages, int variant) {
    return tile_shape(tc).bm * (block_k(dt, tc, stages, variant) * in_size(dt) / kChunk) / threads(tc);
}
constexpr int loads_b(int dt, int tc, int stages, int variant) {
    return tile_shape(tc).bn * (block_k(dt, tc, stages, variant) * in_size(dt) / kChunk) / threads(tc);
}

// XOR swizzle of a K-contiguous row (see the header comment).  It depends
// only on row % 32, so a fragment of 32 rows starting at a multiple of 32
// has the same per-lane swizzle wherever it sits in the tile.  For 128-byte
// rows (two per 256-byte bank line) it takes row bits 1, 3, 2 as its bits
// 0, 1, 2.  One clock of the 16x16 read takes chunk c of rows 0-3 and 12-15
// and chunk c ^ 1 of rows 4-11 (of each 16); for the even rows of those the
// swizzle gives c ^ {0, 1, 6, 7} and c ^ {5, 4, 3, 2}, all different (odd
// rows alike, in the other half of the banks).  The earlier
// (row & 7) ^ ((row >> 3) & 3) served the 32x32 read alone and cost the
// 16x16 read 4 extra clocks.
constexpr int swz(int cpr, int row) {
    return cpr >= 16 ? (row & 15)
         : cpr == 8  ? (((row >> 1) & 1) | (((row >> 3) & 1) << 1) | (((row >> 2) & 1) << 2))
         : cpr == 4  ? ((row >> 2) & 3)
                     : 0;
}
// Row-major (K x N) B tile of layout RR: BK rows of N-contiguous data.  Its
// MFMA fragments are read with gfx950's transposing LDS reads: within each
// group of 16 lanes, every lane supplies the address of 8 bytes (4 fp16/bf16
// or 8 int8 elements along N) from one of 4 (fp16/bf16) or 8 (int8)
// consecutive K rows, and each lane receives the elements of one N column
// from those rows -- the lane layout was measured with a probe:
//   16-bit: out lane i, element e <- row-piece of lane 4e + i/4, element i%4
//   8-bit:  out lane i, element e <- row-piece of lane 2e + i/8, element i%8.
// Two such groups (32 lanes, 256 bytes) are served per clock and together
// read 64 (16-bit) or 32 (8-bit) bytes from each of those rows.  The
// swizzle below XORs the 16-byte chunk index of a row with a function of the
// row so that these 4 or 8 row pieces land in different banks.  fp32 B
// fragments are gathered element by element and are not swizzled.
constexpr int rr_rows_per_read(int dt) { return dt == DT_I8 ? 8 : 4; }
// The (k row, n column) of the 8-byte piece lane l supplies to the first
// transposing read of a B fragment, relative to the fragment's first column
// and the step's first k row.  32x32 blocks: half-wave h = l / 32 takes k
// rows from 8 h (16-bit types) / 16 h (int8), 16-lane groups g = l / 16
// alternate between the fragment's two 16-column halves; 16x16 blocks: each
// group g takes the fragment's 16 columns at its own k chunk, rows 8 g /
// 16 g on.  The second read of the pair is rr_rows_per_read rows further.
constexpr int rr_lane_k(int dt, bool b16, int l) {
    return dt == DT_I8 ? (b16 ? 16 * (l >> 4) : 16 * (l >> 5)) + (l & 15) / 2
                       : (b16 ? 8 * (l >> 4) : 8 * (l >> 5)) + (l & 15) / 4;
}
constexpr int rr_lane_n(int dt, bool b16, int l) {
    return (b16 ? 0 : 16 * ((l >> 4) & 1)) + (dt == DT_I8 ? 8 * (l & 1) : 4 * (l & 3));
}
constexpr int rr_piece_bytes(int dt) { return dt == DT_I8 ? 32 : 64; }
//
// The transposing read is served in 2 clocks of 32 lanes (lanes 0-31, then
// 32-63; measured).  With 16x16 MFMA blocks the two 16-lane groups of one
// clock read the same 16 columns at k rows 2 * rr_rows_per_read apart (k
// rows 0-3 and 8-11 for 16-bit types, 0-7 and 16-23 for 8-bit), which the
// term above maps to the same banks; for rows of 256 bytes or more a second
// term, in that k bit, moves the second group by half a row piece.  Every
// clock of the 32x32 read takes k rows with equal bits there, so it stays
// conflict-free.
constexpr int swz_rr(int dt, int row_bytes, int k) {
    return dt == DT_F32 ? 0
         : ((k / (row_bytes >= 256 ? 1 : 256 / row_bytes))
            % (rr_rows_per_read(dt) / (row_bytes >= 256 ? 1 : 256 / row_bytes) > 0
                   ? rr_rows_per_read(dt) / (row_bytes >= 256 ? 1 : 256 / row_bytes) : 1))
               * (rr_piece_bytes(dt) / kChunk)
           ^ (row_bytes >= 256 ? ((k / (2 * rr_rows_per_read(dt))) & 1) * (rr_piece_bytes(dt) / kChunk / 2) : 0);
}

// Epilogue strip of 2-byte outputs: 32 rows of a wave's block, each row
// `cprs` (16, 8 or 4) 16-byte chunks, no padding, written and read in whole
// chunks (ds_write_b128 / ds_read_b128).  The strip is a run of 256-byte
// bank lines (16 slots of 16 bytes), 16 / cprs rows per line.  Measured on
// gfx950 (lds_layout_probe): a 16-byte write is served 8 consecutive lanes
// per clock, and the clock is conflict-free when their 8 chunks fill one
// 128-byte half of the line's slots (slots 0-7 or 8-15) -- 8 distinct slots
// spread over both halves still cost a cycle; a 16-byte read 16 lanes per
// clock (lanes 2 (l / 32) + the parity of bits 2-4 of l), conflict-free when
// they reach 16 different slots.  The writes put 8 consecutive rows' copies
// of one chunk index in a clock; the read-back reads whole rows.
// strip_off gives the byte offset of chunk c of row r so that both are
// conflict-free (checked on the host against these models and measured):
//   cprs 16: one row per line, chunk c ^ (r mod 16);
//   cprs 8:  rows 2m, 2m+1 share line m; chunks 0-3 in the first half,
//            4-7 in the second, slot 2 ((c mod 4) ^ (m mod 4)) + (r mod 2);
//   cprs 4:  rows 4m .. 4m+3 share line m; chunks 0-1 in the first half,
//            2-3 in the second, slot (2 (r mod 4) + (c mod 2)) ^ (m mod 2).
// The 16-byte chunk each lane writes once the epilogue's lane swap has
// paired its 8-byte pieces: 16x16 blocks, pair pb of blocks (2 pb, 2 pb + 1),
// 16-lane group g (columns 8 (g / 2) .. +7 of block 2 pb + g % 2); 32x32
// blocks, block fn, step pair j (steps 2j, 2j+1), half-wave h.
constexpr int epi16_chunk(int pb, int g) { return 4 * pb + 2 * (g & 1) + (g >> 1); }
constexpr int epi32_chunk(int fn, int j, int h) { return 4 * fn + 2 * j + h; }
constexpr int strip_off(int cprs, int row, int c) {
    return cprs == 16 ? row * 256 + ((c ^ (row & 15)) * 16)
         : cprs == 8  ? (row >> 1) * 256 + (8 * (c >> 2) + 2 * ((c & 3) ^ ((row >> 1) & 3)) + (row & 1)) * 16
                      : (row >> 2) * 256 + (8 * (c >> 1) + (((row & 3) * 2 + (c & 1)) ^ ((row >> 2) & 1))) * 16;
}

// Physical chunk index (within the tile) of logical (row, chunk).
constexpr int phys_chunk(int cpr, int row, int chunk) { return row * cpr + (chunk ^ swz(cpr, row)); }
// Logical chunk that physical chunk p holds (the inverse of the above).
constexpr int logical_row(int cpr, int p) { return p / cpr; }
constexpr int logical_chunk(int cpr, int p) { return (p % cpr) ^ swz(cpr, p / cpr); }

// K-tile order of the K loop.  When K is not a multiple of bkmax (the
// K-tile of the class's 1-2 stage instances), the `head` tiles covering the
// K columns past the last multiple of bkmax -- the last of them ragged --
// come first, in order; the other `nbody` tiles follow in order, starting
// at tile `rot` and wrapping around.  Logical tile t is physical tile
// k_phys_tile(t, ...).
constexpr int k_head_tiles(int K, int bk, int bkmax) { return (K % bkmax + bk - 1) / bk; }
constexpr int k_phys_tile(int t, int head, int nbody, int rot) {
    return t < head ? nbody + t : (t - head + rot >= nbody ? t - head + rot - nbody : t - head + rot);
}

// Stream-K schedule.  The last `sk_tiles` C tiles of a call are cut into
// units (the class's largest K-tile; a K shorter than one unit is one
// unit), numbered tile by tile, `total` = sk_tiles x units; workgroup g of
// G (G <= total) takes units [sk_begin(g), sk_begin(g + 1)).  Its piece of
// each tile it touches is contiguous.  A tile that several workgroups touch
// is summed from partial tiles: workgroup g writes the piece that begins
// its range into partial slot 2g, and a piece that begins at a tile's first
// unit (and ends inside that tile: the last piece of its range) into slot
// 2g + 1.  A piece that is a whole tile is stored as C directly.
constexpr int64_t sk_begin(int64_t g, int64_t G, int64_t total) { return g * total / G; }
// The workgroup whose range holds unit i (the largest g with sk_begin(g) <= i).
constexpr int64_t sk_owner(int64_t i, int64_t G, int64_t total) { return ((i + 1) * G + total - 1) / total - 1; }
// End (a unit of its tile, at most U) of the piece of range [i, e) that
// starts at unit i: the piece covers units i mod U .. sk_piece_end - 1 of
// tile i / U.
constexpr int64_t sk_piece_end(int64_t i, int64_t e, int64_t U) {
    return (i % U + (e - i) < U) ? i % U + (e - i) : U;
}
// Partial slot of workgroup g's piece of the tile whose first unit is t0.
constexpr int64_t sk_slot(int64_t g, int64_t t0, int64_t G, int64_t total) {
    return 2 * g + (sk_begin(g, G, total) >= t0 ? 0 : 1);
}

// Budget check of one instance: LDS ring within the CU's LDS, and every
// per-lane load count a whole number.
constexpr bool instance_fits(int dt, int tc, int stages, int variant) {
    return stages >= 1 && stages <= kMaxStages
        && lds_bytes(dt, tc, stages, variant) <= kLdsBudget
        && (tile_shape(tc).bm * cpr_k(tc, stages, variant)) % threads(tc) == 0
        && (tile_shape(tc).bn * cpr_k(tc, stages, variant)) % threads(tc) == 0
        && loads_a(dt, tc, stages, variant) >= 1 && loads_b(dt, tc, stages, variant) >= 1;
}

}  // namespace pg

#endif
