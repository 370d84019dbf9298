// lds_layout_probe.hip -- LDS bank conflicts of the GEMM's fragment reads
// under three tile layouts: rows as they come (none), rows padded by 16 bytes
// (pad), and the XOR swizzle the kernels use (xor).  The padding/swizzling
// study is the next step the pipelining study names for its shared-memory
// conflicts; here it is measured on gfx950 with SQ_LDS_BANK_CONFLICT.
//
// Each dispatch runs one pattern: one wave repeats a single 64-lane read
// (ds_read_b128 for the K-contiguous fragments of layout RC, the transposing
// ds_read_b64_tr_b16 for layout RR's N-contiguous B tile) 256 times; the
// per-lane byte offsets come from a table built on the host exactly as the
// kernels form them.  Patterns rc_* are the read of the 32x32 MFMA blocks
// (lane l: row l % 32, chunk c0 + l / 32); rc16* that of the 16x16 blocks
// (lane l: row 16 h + l % 16, chunk c0 + l / 16).  The pair_i_j patterns
// find which lanes one clock of a 16-byte read serves together: only lanes
// i and j are active and read the same bank group 256 bytes apart, so the
// read conflicts exactly when the two lanes share a clock; trpair_i_j does
// the same for the transposing read with every lane active (the others read
// one broadcast piece).  Run it under
//   rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS -- ./lds_layout_probe
// and read the counters dispatch by dispatch in the order it prints.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <string>
#include <vector>

#include "tile_layout.h"

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
#define LDSP __attribute__((address_space(3)))

constexpr int kBytes = 65536;
constexpr int kReps = 256;

template <int TR>
__global__ void __launch_bounds__(64) probe(const int* __restrict__ offs, int* out) {
    __shared__ __attribute__((aligned(16))) unsigned char raw[kBytes];
    for (int i = threadIdx.x; i < kBytes / 16; i += 64) ((i32x4 LDSP*)raw)[i] = i32x4{i, i, i, i};
    __syncthreads();
    const int t = offs[threadIdx.x];                    // < 0: the lane takes no part
    const int o = t & (kBytes - (TR ? 8 : 16));         // keeps every read inside the buffer, aligned
    int acc = 0;
    for (int r = 0; r < (t >= 0 ? kReps : 0); ++r) {
        if constexpr (TR) {
            const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 LDSP*)(raw + o));
            acc += v[0] ^ v[3];
        } else {
            const i32x4 v = *(volatile i32x4 LDSP*)(raw + o);
            acc += v[0] ^ v[3];
        }
        __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));   // one read in flight
    }
    out[threadIdx.x] = acc;
}

struct Pattern {
    std::string name;
    bool tr;
    std::vector<int> off;
};

}  // namespace

int main() {
    using namespace pg;
    std::vector<Pattern> pats;
    // Layout RC: lane l reads row l % 32 at logical chunk c0 + l / 32 of a
    // tile with cpr 16-byte chunks per row (c0 = 2, a mid-tile step).
    for (int cpr : {4, 8, 16}) {
        for (int lay = 0; lay < 3; ++lay) {
            Pattern p{"rc_cpr" + std::to_string(cpr) + (lay == 0 ? "_none" : lay == 1 ? "_pad16" : "_xor"), false, {}};
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
            Pattern p{"rc16h" + std::to_string(h) + "_cpr8" + ln[lay], false, {}};
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
        Pattern p{"rc_cpr8_xorprev", false, {}};
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
        Pattern p{std::string("rr_tr16_rows512") + (lay == 0 ? "_none" : lay == 1 ? "_pad16" : "_xor"), true, {}};
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
            Pattern p{"pair_" + std::to_string(i) + "_" + std::to_string(j), false, std::vector<int>(64, -1)};
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
        Pattern p{std::string("rr16_tr16_rows512") + (lay == 0 ? "_xor" : "_xorprev"), true, {}};
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
            Pattern p{"trpair_" + std::to_string(i) + "_" + std::to_string(j), true, std::vector<int>(64, 8)};
            p.off[i] = 0;
            p.off[j] = 512;
            pats.push_back(p);
        }
    {
        Pattern p{"trpair_none", true, std::vector<int>(64, 8)};   // the broadcast alone
        pats.push_back(p);
    }

    int *d_off, *d_out;
    if (hipMalloc(&d_off, 64 * sizeof(int)) != hipSuccess || hipMalloc(&d_out, 64 * sizeof(int)) != hipSuccess) return 1;
    for (size_t i = 0; i < pats.size(); ++i) {
        for (int o : pats[i].off)
            if (o < -1 || o + 16 > kBytes) { std::printf("offset out of range in %s\n", pats[i].name.c_str()); return 1; }
        if (hipMemcpy(d_off, pats[i].off.data(), 64 * sizeof(int), hipMemcpyHostToDevice) != hipSuccess) return 1;
        if (pats[i].tr)
            hipLaunchKernelGGL(probe<1>, dim3(1), dim3(64), 0, 0, d_off, d_out);
        else
            hipLaunchKernelGGL(probe<0>, dim3(1), dim3(64), 0, 0, d_off, d_out);
        if (hipDeviceSynchronize() != hipSuccess) return 1;
        std::printf("dispatch %zu: %s (%d reads)\n", i, pats[i].name.c_str(), kReps);
    }
    return 0;
}
