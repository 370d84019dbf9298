// lds_layout_probe.hip -- LDS bank conflicts of the GEMM's fragment reads
// under three tile layouts: rows as they come (none), rows padded by 16 bytes
// (pad), and the XOR swizzle the kernels use (xor); the lane grouping of the
// LDS accesses the kernels issue (16-byte reads, transposing reads, 8- and
// 16-byte writes); and the epilogue's staging strips of 2-byte outputs.  The
// padding/swizzling study is the next step the pipelining study names for
// its shared-memory conflicts; here it is measured on gfx950 with
// SQ_LDS_BANK_CONFLICT.
//
// Each dispatch runs one pattern: one wave repeats a single 64-lane access
// (ds_read_b128 for the K-contiguous fragments of layout RC, the transposing
// ds_read_b64_tr_b16 for layout RR's N-contiguous B tile, ds_write2_b64 /
// ds_write_b64 / ds_write_b128 for the epilogue) 256 times; the per-lane
// byte offsets come from a table built on the host exactly as the kernels
// form them.  Patterns rc_* are the read of the 32x32 MFMA blocks
// (lane l: row l % 32, chunk c0 + l / 32); rc16* that of the 16x16 blocks
// (lane l: row 16 h + l % 16, chunk c0 + l / 16).  The pair_i_j patterns
// (and w2pair / w1pair / wqpair for the writes) find which lanes one clock
// serves together: only lanes i and j are active and touch the same bank
// group 256 bytes apart, so the access conflicts exactly when the two lanes
// share a clock; trpair_i_j does the same for the transposing read with every
// lane active (the others read one broadcast piece).  epi* and epq* are the
// epilogue strips: the earlier 8-byte layouts, and the 16-byte pieces the
// epilogue writes now, placed by strip_off (tile_layout.h).  Run it under
//   rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS -- ./lds_layout_probe
// and read the counters dispatch by dispatch in the order it prints (the
// offset-table copies between them are dispatches of their own).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <string>
#include <vector>

#include "tile_layout.h"

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
#define LDSP __attribute__((address_space(3)))

constexpr int kBytes = 65536;
constexpr int kReps = 256;

// MODE 0: ds_read_b128; 1: the transposing ds_read_b64_tr_b16; 2: the
// epilogue's paired 8-byte write (two 8-byte pieces 32 bytes apart, one
// ds_write2_b64); 3: one 8-byte write (ds_write_b64); 4: one 16-byte write
// (ds_write_b128).
template <int MODE>
__global__ void __launch_bounds__(64) probe(const int* __restrict__ offs, int* out) {
    __shared__ __attribute__((aligned(16))) unsigned char raw[kBytes];
    for (int i = threadIdx.x; i < kBytes / 16; i += 64) ((i32x4 LDSP*)raw)[i] = i32x4{i, i, i, i};
    __syncthreads();
    const int t = offs[threadIdx.x];                    // < 0: the lane takes no part
    // keeps every access inside the buffer (MODE 2: both pieces in its
    // first half) and aligned
    const int o = MODE == 0 ? t & (kBytes - 16) : MODE == 1 ? t & (kBytes - 8)
                : MODE == 4 ? t & (kBytes / 2 - 16) : t & (kBytes / 2 - 8);
    static_assert(MODE >= 0 && MODE <= 4, "probe mode");
    int acc = 0;
    for (int r = 0; r < (t >= 0 ? kReps : 0); ++r) {
        if constexpr (MODE == 1) {
            const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 LDSP*)(raw + o));
            acc += v[0] ^ v[3];
        } else if constexpr (MODE == 2) {
            // written as the instruction itself: the compiler would drop or
            // split stores that nothing reads (both pieces stay inside the
            // buffer, see o)
            const i32x2 v = {r, acc};
            const uint32_t a = (uint32_t)(uintptr_t)(raw + o);
            asm volatile("ds_write2_b64 %0, %1, %1 offset1:4" ::"v"(a), "v"(v) : "memory");
            acc += 1;
        } else if constexpr (MODE == 3) {
            const i32x2 v = {r, acc};
            const uint32_t a = (uint32_t)(uintptr_t)(raw + o);
            asm volatile("ds_write_b64 %0, %1" ::"v"(a), "v"(v) : "memory");
            acc += 1;
        } else if constexpr (MODE == 4) {
            const i32x4 v = {r, acc, r, acc};
            const uint32_t a = (uint32_t)(uintptr_t)(raw + o);
            asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(v) : "memory");
            acc += 1;
        } else {
            const i32x4 v = *(volatile i32x4 LDSP*)(raw + o);
            acc += v[0] ^ v[3];
        }
        __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));   // one access in flight
    }
    out[threadIdx.x] = acc;
}

struct Pattern {
    std::string name;
    int mode;   // the probe<MODE> that runs it
    std::vector<int> off;
};

// Candidate layouts of a 32-row strip of 2-byte outputs, 256 bytes of data
// per row: off(row, byte) is where byte `byte` of the row's data goes.
struct EpiLayout {
    std::string name;
    int kind;
    bool paired;   // blocks fn and fn + 1 stay 32 bytes apart (one paired write)
    int off(int row, int b) const {
        const int c = b / 16, w = b % 16;
        switch (kind) {
        case 0: {   // 288-byte rows, 8-byte halves swapped in rows 8-15 and 24-31 (as before)
            const int hs = ((w / 8) ^ ((row >> 3) & 1));
            return row * 288 + c * 16 + 8 * hs + w % 8;
        }
        case 1:     // 272-byte rows
            return row * 272 + b;
        case 2:     // 256-byte rows, chunk XOR (row mod 16)
            return row * 256 + ((c ^ (row & 15)) * 16) + w;
        default:    // 256-byte rows, chunk XOR (row mod 16), halves swapped in rows 16-31
            return row * 256 + ((c ^ (row & 15)) * 16) + 8 * ((w / 8) ^ ((row >> 4) & 1)) + w % 8;
        }
    }
};

std::vector<EpiLayout> epi_layouts() {
    return {{"pad288swap", 0, true}, {"pad272", 1, true}, {"xor256", 2, false}, {"xor256swap", 3, false}};
}

}  // namespace

int main() {
    using namespace pg;
    std::vector<Pattern> pats;
    // Layout RC: lane l reads row l % 32 at logical chunk c0 + l / 32 of a
    // tile with cpr 16-byte chunks per row (c0 = 2, a mid-tile step).
    for (int cpr : {4, 8, 16}) {
        for (int lay = 0; lay < 3; ++lay) {
            Pattern p{"rc_cpr" + std::to_string(cpr) + (lay == 0 ? "_none" : lay == 1 ? "_pad16" : "_xor"), 0, {}};
            for (int l = 0; l < 64; ++l) {
                const int row = l % 32, chunk = 2 + l / 32;
                const int off = lay == 0 ? (row * cpr + chunk) * 16
                              : lay == 1 ? row * (cpr * 16 + 16) + chunk * 16
                                         : phys_chunk(cpr, row, chunk) * 16;
                p.off.push_back(off);
            }
            pats.push_back(p);
        }
    }
    // The 16x16 blocks' read at chunk c0 = 4 of a 128-byte-row tile, for
    // both 16-row halves of a 32-row group.  xorprev: the row swizzle the
    // 128-byte rows had before, (row & 7) ^ ((row >> 3) & 3), conflict-free
    // for the 32x32 read (also measured here) but not for this one.
    auto prev8 = [](int row) { return (row & 7) ^ ((row >> 3) & 3); };
    for (int h = 0; h < 2; ++h) {
        for (int lay = 0; lay < 4; ++lay) {
            const char* ln[] = {"_none", "_pad16", "_xor", "_xorprev"};
            Pattern p{"rc16h" + std::to_string(h) + "_cpr8" + ln[lay], 0, {}};
            for (int l = 0; l < 64; ++l) {
                const int row = 16 * h + l % 16, chunk = 4 + l / 16, cpr = 8;
                const int off = lay == 0 ? (row * cpr + chunk) * 16
                              : lay == 1 ? row * (cpr * 16 + 16) + chunk * 16
                              : lay == 2 ? phys_chunk(cpr, row, chunk) * 16
                                         : (row * cpr + (chunk ^ prev8(row))) * 16;
                p.off.push_back(off);
            }
            pats.push_back(p);
        }
    }
    {
        Pattern p{"rc_cpr8_xorprev", 0, {}};
        for (int l = 0; l < 64; ++l) {
            const int row = l % 32, chunk = 2 + l / 32;
            p.off.push_back((row * 8 + (chunk ^ prev8(row))) * 16);
        }
        pats.push_back(p);
    }
    // Layout RR, bf16 B tile of the 256x256 class (512-byte rows): lane j of
    // 16-lane group g addresses 8 bytes of row k at column n (step 1, read 0).
    for (int lay = 0; lay < 3; ++lay) {
        const int rb = 512;
        Pattern p{std::string("rr_tr16_rows512") + (lay == 0 ? "_none" : lay == 1 ? "_pad16" : "_xor"), 1, {}};
        for (int l = 0; l < 64; ++l) {
            const int h = l / 32, g = l / 16, j = l % 16;
            const int k = 16 + 8 * h + j / 4, n = 16 * (g & 1) + 4 * (j & 3);
            const int c = n * 2 / 16, b = n * 2 % 16;
            const int off = lay == 0 ? k * rb + c * 16 + b
                          : lay == 1 ? k * (rb + 16) + c * 16 + b
                                     : k * rb + (c ^ swz_rr(DT_BF16, rb, k)) * 16 + b;
            p.off.push_back(off);
        }
        pats.push_back(p);
    }

    // lane pairs: lane i reads byte 0, lane j byte 256 (bank group 0 of the
    // next 256-byte line), every other lane is off
    for (int i = 0; i < 64; i += 8)
        for (int j = 0; j < 64; ++j) {
            if (j == i) continue;
            Pattern p{"pair_" + std::to_string(i) + "_" + std::to_string(j), 0, std::vector<int>(64, -1)};
            p.off[i] = 0;
            p.off[j] = 256;
            pats.push_back(p);
        }

    // The 16x16 blocks' B read of layout RR (bf16, 512-byte rows) under the
    // kernels' RR swizzle: each 16-lane group g takes the same 16 columns at
    // its own k rows 8g + j/4 (j = lane % 16), where the 32x32 read (above)
    // splits the columns between groups and the k rows between half-waves.
    // xorprev: the earlier RR swizzle of these rows, (k mod 4) x 4 chunks.
    for (int lay = 0; lay < 2; ++lay) {
        const int rb = 512;
        Pattern p{std::string("rr16_tr16_rows512") + (lay == 0 ? "_xor" : "_xorprev"), 1, {}};
        for (int l = 0; l < 64; ++l) {
            const int g = l / 16, j = l % 16;
            const int k = 8 * g + j / 4, n = 16 + 4 * (j & 3);
            const int c = n * 2 / 16, b = n * 2 % 16;
            const int x = lay == 0 ? swz_rr(DT_BF16, rb, k) : (k % 4) * 4;
            p.off.push_back(k * rb + (c ^ x) * 16 + b);
        }
        pats.push_back(p);
    }
    // Lane pairs of the transposing read: every lane active; all but lanes i
    // and j read one 8-byte piece (a broadcast, bytes 8-15); lane i reads
    // bytes 0-7, lane j bytes 512-519 (the same banks, 512 bytes on).
    for (int i = 0; i < 64; i += 16)
        for (int j = 0; j < 64; ++j) {
            if (j == i) continue;
            Pattern p{"trpair_" + std::to_string(i) + "_" + std::to_string(j), 1, std::vector<int>(64, 8)};
            p.off[i] = 0;
            p.off[j] = 512;
            pats.push_back(p);
        }
    {
        Pattern p{"trpair_none", 1, std::vector<int>(64, 8)};   // the broadcast alone
        pats.push_back(p);
    }

    // Paired 8-byte writes (the epilogue's ds_write2_b64: pieces at o and
    // o + 32): which lanes one clock serves together.  w2pair_i_j: only
    // lanes i and j write, lane i at byte 0, lane j at byte 256 (both pieces
    // on the same banks as lane i's); w2cross_i_j: lane j at byte 224, so
    // only its second piece meets lane i's first.
    for (int i : {0, 1, 4, 8, 16, 32})
        for (int j = 0; j < 64; ++j) {
            if (j == i) continue;
            Pattern p{"w2pair_" + std::to_string(i) + "_" + std::to_string(j), 2, std::vector<int>(64, -1)};
            p.off[i] = 0;
            p.off[j] = 256;
            pats.push_back(p);
        }
    for (int j = 1; j < 64; ++j) {
        Pattern p{"w2cross_0_" + std::to_string(j), 2, std::vector<int>(64, -1)};
        p.off[0] = 0;
        p.off[j] = 224;
        pats.push_back(p);
    }
    {
        Pattern p{"w2single_0", 2, std::vector<int>(64, -1)};   // one lane alone
        p.off[0] = 0;
        pats.push_back(p);
    }
    // Single 8-byte writes (ds_write_b64): lane pairs as above.
    for (int i : {0, 4, 16, 32})
        for (int j = 0; j < 64; ++j) {
            if (j == i) continue;
            Pattern p{"w1pair_" + std::to_string(i) + "_" + std::to_string(j), 3, std::vector<int>(64, -1)};
            p.off[i] = 0;
            p.off[j] = 256;
            pats.push_back(p);
        }
    // Single 16-byte writes (ds_write_b128): lane pairs as above.
    for (int i : {0, 4, 16, 32})
        for (int j = 0; j < 64; ++j) {
            if (j == i) continue;
            Pattern p{"wqpair_" + std::to_string(i) + "_" + std::to_string(j), 4, std::vector<int>(64, -1)};
            p.off[i] = 0;
            p.off[j] = 256;
            pats.push_back(p);
        }
    // Strips of 16-byte pieces (each lane one 16-byte chunk of a row, as
    // the epilogue holds them once lane swaps have paired its 8-byte
    // pieces), rows of cprs chunks placed by strip_off: the 16x16 blocks'
    // write (lane l: row 16 h + l % 16, chunk 2 (g % 2) + g / 2 with
    // g = l / 16), the 32x32 blocks' write (row l % 32, chunk c0 + l / 32)
    // and the row-contiguous read-back.  xorsw: chunk c ^ (the row's 256-byte
    // line mod cprs), conflict-free for the reads but not for the 8-lane
    // write clocks of 128- and 64-byte rows.
    auto xorsw = [](int cprs, int row, int c) {
        return row * cprs * 16 + (c ^ (((row * cprs) >> 4) & (cprs - 1))) * 16;
    };
    for (int lay = 0; lay < 2; ++lay)
        for (int cprs : {16, 8, 4}) {
            const std::string cs = std::string(lay == 0 ? "_stripoff" : "_xorsw") + "_cprs" + std::to_string(cprs);
            auto off = [&](int row, int c) { return lay == 0 ? strip_off(cprs, row, c) : xorsw(cprs, row, c); };
            if (cprs == 16)
                for (int h = 0; h < 2; ++h) {
                    Pattern p{"epq16w_h" + std::to_string(h) + cs, 4, {}};
                    for (int l = 0; l < 64; ++l) {
                        const int row = 16 * h + l % 16, g = l / 16;
                        p.off.push_back(off(row, 2 * (g & 1) + (g >> 1)));
                    }
                    pats.push_back(p);
                }
            for (int c0 = 0; c0 < cprs; c0 += 2) {
                Pattern p{"epq32w_c" + std::to_string(c0) + cs, 4, {}};
                for (int l = 0; l < 64; ++l) p.off.push_back(off(l % 32, c0 + l / 32));
                pats.push_back(p);
            }
            for (int i = 0; i < 32 / (64 / cprs); ++i) {
                Pattern p{"epqr_i" + std::to_string(i) + cs, 0, {}};
                for (int l = 0; l < 64; ++l) p.off.push_back(off((64 / cprs) * i + l / cprs, l % cprs));
                pats.push_back(p);
            }
        }
    // The epilogue strips of 2-byte outputs as the kernels write and read
    // them (16x16 blocks: lane l holds row 16 h + l % 16, columns
    // 16 fn + 4 (l / 16) .. +3, and writes blocks fn and fn + 1 together;
    // 32x32 blocks: lane l holds row l % 32, columns 32 fn + 8 q + 4 (l / 32)
    // .. +3, blocks q and q + 2... as the compiler pairs them) and read back
    // row-contiguously (16 lanes per 256-byte row).
    for (const EpiLayout& L : epi_layouts()) {
        // 16x16 blocks: write of blocks fn = 0 (and 1, paired when the
        // layout keeps them 32 bytes apart), for both 16-row halves
        for (int h = 0; h < 2; ++h)
            for (int fn = 0; fn < (L.paired ? 1 : 2); ++fn) {
                Pattern p{"epi16w_h" + std::to_string(h) + "_fn" + std::to_string(fn) + "_" + L.name,
                          L.paired ? 2 : 3, {}};
                for (int l = 0; l < 64; ++l) p.off.push_back(L.off(16 * h + l % 16, 32 * fn + 8 * (l / 16)));
                pats.push_back(p);
            }
        // 32x32 blocks: write of q = 0 (and 1) of block fn = 0
        for (int q = 0; q < (L.paired ? 1 : 2); ++q) {
            Pattern p{"epi32w_q" + std::to_string(q) + "_" + L.name, L.paired ? 2 : 3, {}};
            for (int l = 0; l < 64; ++l) p.off.push_back(L.off(l % 32, 16 * q + 8 * (l / 32)));
            pats.push_back(p);
        }
        // read-back: 16 lanes per row, rows 4 i .. 4 i + 3
        for (int i = 0; i < 2; ++i) {
            Pattern p{"epir_i" + std::to_string(i) + "_" + L.name, 0, {}};
            for (int l = 0; l < 64; ++l) p.off.push_back(L.off(4 * i + l / 16, 16 * (l % 16)) & ~15);
            pats.push_back(p);
        }
    }

    int *d_off, *d_out;
    if (hipMalloc(&d_off, 64 * sizeof(int)) != hipSuccess || hipMalloc(&d_out, 64 * sizeof(int)) != hipSuccess) return 1;
    for (size_t i = 0; i < pats.size(); ++i) {
        for (int o : pats[i].off)
            if (o < -1 || o + 16 > kBytes || (pats[i].mode >= 2 && o + 40 > kBytes / 2) ||
                (pats[i].mode == 4 && o >= 0 && (o & 15) != 0)) {
                std::printf("offset out of range in %s\n", pats[i].name.c_str());
                return 1;
            }
        if (hipMemcpy(d_off, pats[i].off.data(), 64 * sizeof(int), hipMemcpyHostToDevice) != hipSuccess) return 1;
        if (pats[i].mode == 1)
            hipLaunchKernelGGL(probe<1>, dim3(1), dim3(64), 0, 0, d_off, d_out);
        else if (pats[i].mode == 2)
            hipLaunchKernelGGL(probe<2>, dim3(1), dim3(64), 0, 0, d_off, d_out);
        else if (pats[i].mode == 3)
            hipLaunchKernelGGL(probe<3>, dim3(1), dim3(64), 0, 0, d_off, d_out);
        else if (pats[i].mode == 4)
            hipLaunchKernelGGL(probe<4>, dim3(1), dim3(64), 0, 0, d_off, d_out);
        else
            hipLaunchKernelGGL(probe<0>, dim3(1), dim3(64), 0, 0, d_off, d_out);
        if (hipDeviceSynchronize() != hipSuccess) return 1;
        std::printf("dispatch %zu: %s (%d reads)\n", i, pats[i].name.c_str(), kReps);
    }
    return 0;
}
