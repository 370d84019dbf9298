// Host check of tile_layout.h (the header the kernels include):
//  1. the XOR swizzle is a bijection inside every row, and logical_chunk()
//     inverts phys_chunk();
//  2. the fragment reads -- 32x32 blocks: lane l reads row (rb + l % 32) at
//     chunk (c0 + l / 32); 16x16 blocks (128-byte rows): row
//     (rb + 16 h + l % 16) at chunk (c0 + l / 16), c0 a multiple of 4; rb a
//     multiple of 32 -- are free of LDS bank conflicts in gfx950's LDS as
//     measured: 64 banks of 4 bytes, a 16-byte read served in 4 clocks of 16
//     lanes, lane l in clock 2 (l / 32) + parity of bits 2-4 of l (lanes
//     0-3, 12-15, 20-23, 24-27 share a clock), so the 16-byte bank groups
//     (address / 16 mod 16) hit by the lanes of one clock must all differ;
//     the model reproduces the conflict cycles measured for unswizzled,
//     padded and swizzled tiles (checked below);
//  3. without the swizzle the same read does conflict (so 2 is not vacuous);
//  4. the transposing reads of layout RR's B tile are conflict-free;
//  5. the K-tile order is a permutation with the ragged tile in the
//     prologue, and every stage count adds the k-slices in one order;
//  6. the epilogue strips of 2-byte outputs (strip_off) are written with
//     16-byte writes and read back without bank conflicts (the measured
//     8-lane write clocks, the 16-lane read clocks above);
//  7. the stream-K schedule (sk_begin, sk_owner, sk_piece_end, sk_slot),
//     walked as the kernel walks it: every unit of every tile is covered
//     once, a tile is either one whole piece or partial pieces from the
//     consecutive workgroups sk_owner names, in K order, each writing the
//     slot sk_slot gives the finisher, and no two partial pieces share a
//     slot.
// Prints one line per chunks-per-row value; exits non-zero on failure.
#include <cstdio>
#include <initializer_list>
#include "tile_layout.h"

using namespace pg;

// Lane l's clock (0-3) in a 16-byte LDS read, as measured lane pair by lane
// pair with SQ_LDS_BANK_CONFLICT.
static int clock_of(int l) {
    const int b = (l % 32) / 4;
    return 2 * (l / 32) + (((b >> 2) ^ (b >> 1) ^ b) & 1);
}

// Extra clocks of one read whose lane l reads the 16 bytes at offs[l]: per
// clock, the most distinct addresses any bank group is asked for, minus one.
static int extra_clocks(const int (&offs)[64]) {
    int total = 0;
    for (int c = 0; c < 4; ++c) {
        int addr[16][16], n[16] = {0}, worst = 1;
        for (int l = 0; l < 64; ++l) {
            if (clock_of(l) != c) continue;
            const int g = (offs[l] / 16) % 16;
            bool seen = false;
            for (int i = 0; i < n[g]; ++i) seen |= addr[g][i] == offs[l];
            if (!seen) addr[g][n[g]++] = offs[l];
            if (n[g] > worst) worst = n[g];
        }
        total += worst - 1;
    }
    return total;
}

// Byte offsets of a fragment read.  wide: the 32x32 read, else the 16x16
// read with row half h.  lay 0: unswizzled, 1: rows padded by 16 bytes,
// 2: swizzled by swz().
static void read_offsets(int cpr, int lay, bool wide, int rb, int c0, int h, int (&offs)[64]) {
    for (int l = 0; l < 64; ++l) {
        const int row = wide ? rb + (l % 32) : rb + 16 * h + (l % 16);
        const int chunk = wide ? c0 + l / 32 : c0 + l / 16;
        offs[l] = lay == 0 ? (row * cpr + chunk) * 16
                : lay == 1 ? row * (cpr * 16 + 16) + chunk * 16
                           : phys_chunk(cpr, row, chunk) * 16;
    }
}

// Extra clocks of one 16-byte write (ds_write_b128) whose lane l writes
// offs[l] (< 0: lane off).  As measured: 8 consecutive lanes per clock; a
// clock takes one pass per 128-byte half of the 256-byte bank line its
// chunks touch, times the most distinct addresses any 16-byte slot is asked
// for.
static int write_extra_clocks(const int (&offs)[64]) {
    int total = 0;
    for (int k = 0; k < 8; ++k) {
        int addr[16][8], n[16] = {0}, worst = 0;
        bool half[2] = {false, false};
        for (int l = 8 * k; l < 8 * k + 8; ++l) {
            if (offs[l] < 0) continue;
            const int g = (offs[l] / 16) % 16;
            half[g / 8] = true;
            bool seen = false;
            for (int i = 0; i < n[g]; ++i) seen |= addr[g][i] == offs[l];
            if (!seen) addr[g][n[g]++] = offs[l];
            if (n[g] > worst) worst = n[g];
        }
        const int passes = (half[0] ? 1 : 0) + (half[1] ? 1 : 0);
        if (worst > 0) total += passes * worst - 1;
    }
    return total;
}

static int conflict_cycles(int cpr, int lay, bool wide, int rb, int c0, int h) {
    int offs[64];
    read_offsets(cpr, lay, wide, rb, c0, h, offs);
    return extra_clocks(offs);
}

int main() {
    int fail = 0;
    const int cprs[] = {4, 8, 16, 32};
    for (int cpr : cprs) {
        for (int row = 0; row < 512; ++row) {
            bool seen[64] = {false};
            for (int c = 0; c < cpr; ++c) {
                const int p = phys_chunk(cpr, row, c);
                if (p < row * cpr || p >= (row + 1) * cpr || seen[p - row * cpr]) { ++fail; break; }
                seen[p - row * cpr] = true;
                if (logical_row(cpr, p) != row || logical_chunk(cpr, p) != c) ++fail;
            }
            if (swz(cpr, row) != swz(cpr, row % 32)) ++fail;  // depends on row % 32 only
        }
        int worst = 0, raw = 0, worst16 = 0;
        for (int rb = 0; rb < 256; rb += 32) {
            for (int c0 = 0; c0 + 1 < cpr; c0 += 2) {
                int w;
                if ((w = conflict_cycles(cpr, 2, true, rb, c0, 0)) > worst) worst = w;
                if ((w = conflict_cycles(cpr, 0, true, rb, c0, 0)) > raw) raw = w;
            }
            if (cpr == 8)   // the 16x16 blocks read 128-byte rows
                for (int c0 = 0; c0 + 3 < cpr; c0 += 4)
                    for (int h = 0; h < 2; ++h) {
                        const int w = conflict_cycles(cpr, 2, false, rb, c0, h);
                        if (w > worst16) worst16 = w;
                    }
        }
        std::printf("cpr=%d: extra clocks per read: swizzled %d (16x16 read: %d), unswizzled %d\n", cpr, worst,
                    worst16, raw);
        if (worst != 0 || worst16 != 0) ++fail;
        if (raw == 0) ++fail;
    }
    // The model against the conflict cycles measured per read (one wave, the
    // reads at chunk 2 resp. 4): 32x32 read unswizzled 12 / 28 / 60 for
    // 64- / 128- / 256-byte rows and 0 padded; 16x16 read unswizzled 12,
    // padded 4, and 4 under the 128-byte rows' earlier swizzle
    // (row & 7) ^ ((row >> 3) & 3).
    {
        const int cprs3[] = {4, 8, 16}, want[] = {12, 28, 60};
        for (int i = 0; i < 3; ++i)
            if (conflict_cycles(cprs3[i], 0, true, 0, 2, 0) != want[i] ||
                conflict_cycles(cprs3[i], 1, true, 0, 2, 0) != 0) { std::printf("model off: 32x32 cpr %d\n", cprs3[i]); ++fail; }
        for (int h = 0; h < 2; ++h) {
            int prev[64];
            for (int l = 0; l < 64; ++l) {
                const int row = 16 * h + l % 16, chunk = 4 + l / 16;
                prev[l] = (row * 8 + (chunk ^ ((row & 7) ^ ((row >> 3) & 3)))) * 16;
            }
            if (conflict_cycles(8, 0, false, 0, 4, h) != 12 || conflict_cycles(8, 1, false, 0, 4, h) != 4 ||
                extra_clocks(prev) != 4) { std::printf("model off: 16x16 half %d\n", h); ++fail; }
        }
    }
    // Epilogue strips of 2-byte outputs (strip_off, rows of 16, 8 or 4
    // chunks): a one-to-one map onto the strip, and the writes -- 16x16
    // blocks (lane l: row 16 h + l % 16, chunk epi16_chunk(pb, l / 16)),
    // 32x32 blocks (row l % 32, chunk epi32_chunk(fn, j, l / 32)) -- and the
    // row-contiguous read-back conflict-free.  The write model is pinned to
    // the measured counts: lanes i, j of one clock on the same slot 1 extra
    // clock, of different clocks 0; the 32x32 write under the XOR-by-line
    // layout 8 extra clocks for 128- and 64-byte rows, 0 for 256-byte rows.
    {
        int epi_fail = 0;
        for (int cprs : {16, 8, 4}) {
            bool used[32 * 16] = {false};
            for (int row = 0; row < 32; ++row)
                for (int c = 0; c < cprs; ++c) {
                    const int o = strip_off(cprs, row, c);
                    if (o % 16 != 0 || o < 0 || o >= 32 * cprs * 16 || used[o / 16]) ++epi_fail;
                    else used[o / 16] = true;
                }
            int offs[64];
            for (int fn = 0; fn < cprs / 4; ++fn)
                for (int j = 0; j < 2; ++j) {
                    for (int l = 0; l < 64; ++l) offs[l] = strip_off(cprs, l % 32, epi32_chunk(fn, j, l / 32));
                    if (write_extra_clocks(offs) != 0) ++epi_fail;
                }
            if (cprs == 16)
                for (int h = 0; h < 2; ++h)
                    for (int pb = 0; pb < 4; ++pb) {
                        for (int l = 0; l < 64; ++l) offs[l] = strip_off(cprs, 16 * h + l % 16, epi16_chunk(pb, l / 16));
                        if (write_extra_clocks(offs) != 0) ++epi_fail;
                    }
            const int rows_per_read = 64 / cprs;
            for (int i = 0; i < 32 / rows_per_read; ++i) {
                for (int l = 0; l < 64; ++l) offs[l] = strip_off(cprs, rows_per_read * i + l / cprs, l % cprs);
                if (extra_clocks(offs) != 0) ++epi_fail;
            }
            // the measured counts
            for (int c0 = 0; c0 < cprs; c0 += 2) {
                for (int l = 0; l < 64; ++l) {
                    const int row = l % 32;
                    offs[l] = row * cprs * 16 + ((c0 + l / 32) ^ (((row * cprs) >> 4) & (cprs - 1))) * 16;
                }
                if (write_extra_clocks(offs) != (cprs == 16 ? 0 : 8)) { std::printf("write model off: cprs %d\n", cprs); ++epi_fail; }
            }
        }
        for (int i : {0, 4, 16, 32})
            for (int j = 0; j < 64; ++j) {
                if (j == i) continue;
                int offs[64];
                for (int l = 0; l < 64; ++l) offs[l] = -1;
                offs[i] = 0;
                offs[j] = 256;
                if (write_extra_clocks(offs) != (j / 8 == i / 8 ? 1 : 0)) { std::printf("write pair model off: %d %d\n", i, j); ++epi_fail; }
            }
        std::printf("epilogue strips (2-byte outputs): %s\n", epi_fail ? "FAIL" : "one-to-one, writes and read-back conflict-free");
        fail += epi_fail;
    }
    // every instance the library builds fits the LDS budget
    for (int dt = 0; dt < 4; ++dt)
        for (int tc = 0; tc < TILE_COUNT; ++tc)
            for (int s = 1; s <= kMaxStages; ++s)
                for (int v = 0; v < 2; ++v)
                    if (!instance_fits(dt, tc, s, v)) { std::printf("over budget %d %d %d %d\n", dt, tc, s, v); ++fail; }
    // The split ring (3 direct stages at 256x256): three A slots and two B
    // slots of the full K-tile fill the 160 KiB exactly; the register-staged
    // 3-stage instances of the same class halve the K-tile instead.
    for (int dt = 0; dt < 4; ++dt)
        for (int tc = 0; tc < TILE_COUNT; ++tc) {
            const bool big = tc == TILE_L || tc == TILE_W;
            if (split_ring(tc, 3, VAR_DIRECT) != big || split_ring(tc, 3, VAR_REG) || split_ring(tc, 2, VAR_DIRECT) ||
                split_ring(tc, 4, VAR_DIRECT)) ++fail;
            if (big && (block_k(dt, tc, 3, VAR_DIRECT) != block_k(dt, tc, 2, VAR_DIRECT) ||
                        2 * block_k(dt, tc, 3, VAR_REG) != block_k(dt, tc, 2, VAR_REG) ||
                        ring_bytes(dt, tc, 3, VAR_DIRECT) != kLdsBudget)) {
                std::printf("split ring %d %d\n", dt, tc);
                ++fail;
            }
        }
    // Layout RR: the transposing fragment reads of the N-contiguous B tile
    // (lane addresses exactly as the kernel forms them) hit 64 different
    // 4-byte banks in every group of 32 lanes, and the XOR keeps each row a
    // permutation of its chunks; without the XOR they conflict.
    int rr_fail = 0, rr_raw = 1;
    for (int dt = 0; dt < 3; ++dt)
        for (int tc = 0; tc < TILE_COUNT; ++tc) {
            const int sz = in_size(dt), bn = tile_shape(tc).bn, rb = bn * sz, cpr_rr = rb / kChunk;
            const int wtn = bn / tile_shape(tc).wn;
            for (int k = 0; k < 256; ++k) {
                const int x = swz_rr(dt, rb, k);
                if (x < 0 || x >= cpr_rr || (cpr_rr & (cpr_rr - 1)) != 0) ++rr_fail;
            }
            for (int wn = 0; wn < tile_shape(tc).wn; ++wn)
                for (int fn = 0; fn < wtn / 32; ++fn)
                    for (int st = 0; st < 4; ++st)
                        for (int r = 0; r < 2; ++r)
                            for (int sw = 0; sw < 2; ++sw) {
                                int worst = 1;
                                for (int g0 = 0; g0 < 64; g0 += 32) {
                                    int hits[64] = {0};
                                    for (int l = g0; l < g0 + 32; ++l) {
                                        const int nf = wn * wtn + fn * 32;
                                        const int k = st * (dt == DT_I8 ? 32 : 16) + rr_rows_per_read(dt) * r +
                                                      rr_lane_k(dt, false, l);
                                        const int n = nf + rr_lane_n(dt, false, l);
                                        const int c = n * sz / kChunk, b = n * sz % kChunk;
                                        const int addr = k * rb + ((sw ? c ^ swz_rr(dt, rb, k) : c) * kChunk) + b;
                                        for (int w = 0; w < 2; ++w) {
                                            const int bank = (addr / 4 + w) % 64;
                                            if (++hits[bank] > worst) worst = hits[bank];
                                        }
                                    }
                                }
                                if (sw && worst != 1) ++rr_fail;
                                if (!sw && worst > rr_raw) rr_raw = worst;
                            }
        }
    // The 16x16 blocks' RR read (256x256 tile): 16-lane group g takes the
    // fragment's 16 columns at its own k chunk, so one 32-lane clock reads
    // the same columns at two k-row sets; the swizzle keeps it conflict-free.
    {
        const TileShape ts = tile_shape(TILE_L);
        for (int dt = 0; dt < 3; ++dt) {
            const int sz = in_size(dt), rb = ts.bn * sz, wtn = ts.bn / ts.wn;
            for (int wn = 0; wn < ts.wn; ++wn)
                for (int idx = 0; idx < wtn / 16; ++idx)
                    for (int st = 0; st < 2; ++st)
                        for (int r = 0; r < 2; ++r) {
                            int worst = 1;
                            for (int g0 = 0; g0 < 64; g0 += 32) {
                                int hits[64] = {0};
                                for (int l = g0; l < g0 + 32; ++l) {
                                    const int nf = wn * wtn + idx * 16;
                                    const int k = st * (dt == DT_I8 ? 64 : 32) + rr_rows_per_read(dt) * r +
                                                  rr_lane_k(dt, true, l);
                                    const int n = nf + rr_lane_n(dt, true, l);
                                    const int c = n * sz / kChunk, b = n * sz % kChunk;
                                    const int addr = k * rb + (c ^ swz_rr(dt, rb, k)) * kChunk + b;
                                    for (int w = 0; w < 2; ++w) {
                                        const int bank = (addr / 4 + w) % 64;
                                        if (++hits[bank] > worst) worst = hits[bank];
                                    }
                                }
                            }
                            if (worst != 1) { std::printf("RR 16x16 read conflicts: dt %d wn %d idx %d\n", dt, wn, idx); ++rr_fail; }
                        }
        }
    }
    // The lane formulas give each fragment column its k values in MFMA
    // order: the transposing read hands out lane i the piece of the lane
    // that addressed row piece (e * per + i / (16 / per)), element i mod
    // (16 / per)... (16-bit: out lane i, element e <- lane 4e + i/4, element
    // i%4; 8-bit: lane 2e + i/8, element i%8, measured).  So output lane i of
    // a 16-lane group receives column n of its addressing lanes at the k of
    // lanes 4e + i/4 (2e + i/8): consecutive k, the same column for all e.
    for (int dt = 0; dt < 3; ++dt)
        for (int b16 = 0; b16 < 2; ++b16)
            for (int l = 0; l < 64; ++l) {
                const int g0 = l & ~15, i = l & 15, epl = dt == DT_I8 ? 8 : 4;   // elements per lane
                for (int e = 0; e < epl; ++e) {
                    const int src = g0 + (dt == DT_I8 ? 2 * e + i / 8 : 4 * e + i / 4);
                    const int col = rr_lane_n(dt, b16, src) + (dt == DT_I8 ? i % 8 : i % 4);
                    const int col0 = rr_lane_n(dt, b16, g0 + (dt == DT_I8 ? i / 8 : i / 4)) + (dt == DT_I8 ? i % 8 : i % 4);
                    if (col != col0 || rr_lane_k(dt, b16, src) != rr_lane_k(dt, b16, g0 + (dt == DT_I8 ? i / 8 : i / 4)) + e) {
                        std::printf("RR lane formulas: dt %d b16 %d lane %d element %d\n", dt, b16, l, e);
                        ++rr_fail;
                    }
                }
            }
    std::printf("RR transposing reads: swizzled %s, unswizzled worst %d-way\n", rr_fail ? "CONFLICTS" : "conflict-free", rr_raw);
    if (rr_raw == 1) ++rr_fail;
    fail += rr_fail;

    // K-tile order: a permutation of the tiles whose last physical tile (the
    // ragged one) is logical tile head-1, and -- for the classes whose K-tile
    // halves at 3-4 stages -- the same sequence of MFMA k-slices (2 chunks
    // each) at both K-tile sizes, so all stage counts sum in one order.
    int order_fail = 0;
    for (int v = 0; v < 2; ++v)
    for (int dt = 0; dt < 4; ++dt)
        for (int tc = 0; tc < TILE_COUNT; ++tc) {
            const int bkmax = block_k(dt, tc, 1, v), slice = 2 * epc(dt);
            for (int K = 1; K <= 9 * bkmax; K += (K < 3 * bkmax ? 1 : 7)) {
                int seq[2][1024], len[2] = {0, 0};
                for (int s = 1; s <= kMaxStages; ++s) {
                    const int bk = block_k(dt, tc, s, v), nt = (K + bk - 1) / bk;
                    const int head = k_head_tiles(K, bk, bkmax), nbody = nt - head;
                    if (head > (s == 1 ? 1 : s - 1)) ++order_fail;   // head tiles are prologue loads
                    for (int rot = 0; rot < (nbody > 0 ? nbody : 1); rot += 1 + nbody / 5) {
                        bool seen[2048] = {false};
                        for (int t = 0; t < nt; ++t) {
                            const int p = k_phys_tile(t, head, nbody, rot);
                            if (p < 0 || p >= nt || seen[p]) ++order_fail;
                            else seen[p] = true;
                        }
                        if (head > 0 && k_phys_tile(head - 1, head, nbody, rot) != nt - 1) ++order_fail;
                    }
                    if (s != 1 && s != 3) continue;
                    int* q = seq[s == 1 ? 0 : 1];
                    int& n = len[s == 1 ? 0 : 1];
                    for (int t = 0; t < nt; ++t) {
                        const int p = k_phys_tile(t, head, nbody, 0);
                        for (int k0 = p * bk; k0 < (p + 1) * bk; k0 += slice)
                            if (k0 < K && n < 1024) q[n++] = k0;
                    }
                }
                if (len[0] != len[1]) ++order_fail;
                for (int i = 0; i < len[0] && i < len[1]; ++i)
                    if (seq[0][i] != seq[1][i]) { ++order_fail; break; }
            }
        }
    std::printf("K-tile order: %s\n", order_fail ? "FAIL" : "permutation, ragged tile loaded first, one k-slice order for all stage counts");
    fail += order_fail;

    // The kernel's order with K split into P ranges of whole bkmax units
    // (the ragged head with the last split) and each range started at unit
    // rot_u: logical tile t of split p is physical tile tail0 + t for
    // t < head, else tbase + k_phys_tile(t, head, nbody, rot_u * per).
    // Every (P, rot_u): the splits together cover each physical tile once,
    // and the 1-stage and 3-stage K-tiles add the same k-slices in one order.
    int split_fail = 0;
    for (int v = 0; v < 2; ++v)
    for (int dt = 0; dt < 4; ++dt)
        for (int tc = 0; tc < TILE_COUNT; ++tc) {
            const int bkmax = block_k(dt, tc, 1, v), slice = 2 * epc(dt);
            for (int K = 1; K <= 9 * bkmax; K += (K < 3 * bkmax ? 5 : 11))
                for (int P = 1; P <= 3; ++P)
                    for (int rot_u = 0; rot_u < 9; rot_u += 4) {
                        int seq[2][1024], len[2] = {0, 0};
                        for (int si = 0; si < 2; ++si) {
                            const int s = si == 0 ? 1 : 3, bk = block_k(dt, tc, s, v), per = bkmax / bk;
                            const int nt = (K + bk - 1) / bk, units = K / bkmax, head = k_head_tiles(K, bk, bkmax);
                            bool seen[2048] = {false};
                            int covered = 0;
                            for (int p = 0; p < P; ++p) {
                                const int u0 = p * units / P, u1 = (p + 1) * units / P;
                                const int hd = p == P - 1 ? head : 0, nbody = (u1 - u0) * per;
                                const int rot = u1 > u0 ? (rot_u % (u1 - u0)) * per : 0;
                                for (int t = 0; t < nbody + hd; ++t) {
                                    const int q = t < hd ? units * per + t : u0 * per + k_phys_tile(t, hd, nbody, rot);
                                    if (q < 0 || q >= nt || seen[q]) { ++split_fail; continue; }
                                    seen[q] = true;
                                    ++covered;
                                    for (int k0 = q * bk; k0 < (q + 1) * bk; k0 += slice)
                                        if (k0 < K && len[si] < 1024) seq[si][len[si]++] = k0;
                                }
                            }
                            if (covered != nt) ++split_fail;
                        }
                        if (len[0] != len[1]) ++split_fail;
                        for (int i = 0; i < len[0] && i < len[1]; ++i)
                            if (seq[0][i] != seq[1][i]) { ++split_fail; break; }
                    }
        }
    std::printf("K splits and rotation: %s\n", split_fail ? "FAIL" : "every tile once, one k-slice order for all stage counts");
    fail += split_fail;
    // 7. Stream-K schedule.
    int sk_fail = 0;
    long long schedules = 0, partial_tiles = 0;
    for (int64_t tiles = 1; tiles <= 40; tiles += (tiles < 12 ? 1 : 7))
        for (int64_t U = 1; U <= 13; U += (U < 5 ? 1 : 4))
            for (int64_t G = 1; G <= 300; G += (G < 20 ? 1 : 37)) {
                const int64_t total = tiles * U;
                if (G > total) continue;
                ++schedules;
                // pieces[tile] in K order: (workgroup, a, b, slot or -1 for a whole tile)
                struct Piece { int64_t g, a, b, slot; };
                static Piece pieces[40][64];
                int np[40] = {0};
                static bool slot_used[600];
                for (int64_t q = 0; q < 2 * G; ++q) slot_used[q] = false;
                for (int64_t g = 0; g < G; ++g) {
                    const int64_t i0 = sk_begin(g, G, total), e = sk_begin(g + 1, G, total);
                    if (e <= i0) ++sk_fail;   // every range non-empty
                    for (int64_t i = i0; i < e;) {
                        const int64_t t = i / U, a = i - t * U, b = sk_piece_end(i, e, U);
                        if (b <= a || b > U) { ++sk_fail; break; }
                        const bool whole = a == 0 && b == U;
                        const int64_t slot = whole ? -1 : 2 * g + (i == i0 ? 0 : 1);
                        if (np[t] < 64) pieces[t][np[t]++] = Piece{g, a, b, slot};
                        if (!whole) {
                            if (slot_used[slot]) ++sk_fail;
                            slot_used[slot] = true;
                        }
                        i += b - a;
                    }
                }
                for (int64_t t = 0; t < tiles; ++t) {
                    const int64_t t0 = t * U, g0 = sk_owner(t0, G, total), g1 = sk_owner(t0 + U - 1, G, total);
                    int64_t next = 0;
                    for (int k = 0; k < np[t]; ++k) {
                        const Piece& pc = pieces[t][k];
                        if (pc.a != next) ++sk_fail;      // contiguous, in K order
                        next = pc.b;
                        if (pc.g != g0 + k) ++sk_fail;    // the owners, in order
                        if (np[t] > 1 && pc.slot != sk_slot(pc.g, t0, G, total)) ++sk_fail;
                    }
                    if (next != U || np[t] != g1 - g0 + 1) ++sk_fail;
                    if ((np[t] == 1) != (pieces[t][0].slot == -1)) ++sk_fail;
                    partial_tiles += np[t] > 1;
                }
            }
    std::printf("stream-K schedule: %lld schedules, %lld tiles summed from partials: %s\n", schedules,
                partial_tiles, sk_fail ? "FAIL" : "every unit once, owners and slots as the finisher reads them");
    if (partial_tiles == 0) ++sk_fail;
    fail += sk_fail;
    std::printf(fail ? "FAIL (%d)\n" : "OK\n", fail);
    return fail ? 1 : 0;
}
