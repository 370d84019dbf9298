// gemm_kernel.h -- the pipelined tiled GEMM kernel for gfx950 (device code).
//
// C = A * B over BM x BN x BK tiles.  The K loop is split into prologue,
// main loop and drain so that the global->LDS copy of later K-tiles
// overlaps the MFMA work on the current one ("CUDA Kernel Study:
// Pipelining", Case 1 and Case 2; "pipeline-gpu-kernel", step 3).
//
// Two load paths (the pages' ping-pong vs cp.async contrast, Key
// Differences):
//  * DIRECT: buffer loads with the LDS bit set (LDS-DMA): each lane's 16
//    bytes go from memory straight into the LDS slot, no VGPR in between.
//    An LDS ring of STAGES slots; the prologue fills every slot, and at each
//    tile boundary the wave waits with `s_waitcnt vmcnt(n)` until the next
//    tile has landed (vmcnt counts this wave's outstanding loads, which
//    retire in order -- the analogue of cp.async.wait_group), crosses one
//    barrier, and refills the slot every wave has just finished reading.
//    STAGES = 1 is the serial load / sync / compute / sync loop of the
//    README's Background section.  At 3 stages the 256x256 classes split the
//    ring by operand (three A slots, two B slots; see split_ring): the A tile
//    of K-tile kt+2 is loaded while tile kt is multiplied, the B tile of
//    kt+2 right after the barrier that ends tile kt.
//  * REG: buffer loads into VGPR staging sets, then ds_write_b128 into one
//    of two LDS slots (ping-pong).  max(1, STAGES-1) staging sets keep that
//    many tiles in flight in registers; STAGES = 1 is the skill's
//    register-only prefetch into a single LDS buffer (two barriers per
//    iteration), STAGES >= 2 use one barrier per iteration.
// Both paths put a tile in LDS in the same swizzled layout and add the same
// k-slices in the same order, so every (STAGES, variant) pair gives the same
// C.  The 256x256 tile's 2- and 3-stage direct instances build each
// wave's block from 16x16 MFMA blocks instead of 32x32 (a higher sustained
// clock); their results are bit-identical to the 32x32 instances -- exact for
// int8, and measured bit for bit for fp16/bf16 by the GPU tests.
//
// MFMA mapping.  Both operands are read from LDS as one 16-byte chunk per
// lane: lane l takes row (l % 32) of a 32-row fragment and chunk
// (2*step + l/32) of the K-tile.  (The 256x256 instances of the 2-3 stage
// direct ring with K-contiguous B use 16x16 blocks instead; see Block16.)  The B-side fragment is fed as the MFMA's
// first operand and the A-side fragment as its second, so the 32x32 result
// block is C^T and each lane ends up holding four consecutive columns of
// one row of C -- which the epilogue stores as one vector per lane.
// Any k order inside an MFMA is fine as long as both operands use the same
// one, which they do by construction.
//
// Addressing.  Each lane's buffer offset of a chunk is fixed for the whole
// K loop; the K-tile's position goes into the instruction's scalar offset,
// so the loop spends no vector instructions on addresses.  Rows past M (or
// columns past N) read a valid row of the tile instead: they only feed
// outputs that are never stored.  A ragged last K-tile is multiplied first
// (loaded in the prologue; see phys_tile), so it is the only load that
// needs a per-lane test: its chunks past K get an offset beyond the
// buffer's range, and an out-of-range buffer load returns 0 (also into
// LDS).  (When K is not whole 16-byte chunks -- register-staged instances
// of their own -- the chunk holding column K-1 is read in exact pieces; see
// load_k_tail.)  Tiles past the last one get an out-of-range scalar offset
// and load zeros.  Stores are masked.
//
// Split K and stream-K (run, partial): the same kernel, given a split
// count above 1, runs one K range of a C tile per workgroup, or, given
// stream-K tiles, shares their K units out over the grid; the partial tiles
// are combined through a workspace.  With neither it is the plain GEMM.
#ifndef PIPEGEMM_GEMM_KERNEL_H
#define PIPEGEMM_GEMM_KERNEL_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernel_args.h"
#include "tile_layout.h"

namespace pg {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

#define PG_LDS __attribute__((address_space(3)))

// Buffer resource word 3 for gfx9-family raw buffers (32-bit data format,
// no swizzle, no stride).
constexpr int kRsrcWord3 = 0x00020000;
// A buffer offset no valid element reaches: loads from it return zero.
constexpr uint32_t kOob = 0x80000000u;
// Cache-policy operand of a buffer access at device scope (the SC1 bit):
// coherent across the XCDs' L2 caches.
constexpr int kScopeDevice = 16;

template <int DT> struct AccT { typedef f32x16 type; };
template <> struct AccT<DT_I8> { typedef i32x16 type; };
typedef float f32x4 __attribute__((ext_vector_type(4)));

// One 16x16 MFMA block step: acc += X * Y over 4 chunks of k (one 16-byte
// chunk per lane of each operand: 32 k for fp16/bf16, 64 for int8).  The
// matrix cores hold a 0.25-0.3 GHz higher clock on these than on the 32x32
// blocks at the same busy share (measured), and the results are the same
// bits.  Written in place (accumulator tied to the destination): with the
// compiler's own form, the 64 accumulator blocks of a wave moved between
// registers at every K-tile.  The compiler does not see these as MFMAs, so
// the loop that issues them pads the hazards around it itself (Block16).
//   The accumulator is held as four 32-bit words of either type (fp32 bits
// for fp16/bf16): typed as float vectors, the compiler kept them in arch
// VGPRs around the statements that tie them (below) and spilled.
template <int DT>
__device__ __forceinline__ i32x4 mfma16(i32x4 x, i32x4 y, i32x4 c) {
    if constexpr (DT == DT_BF16) {
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(x), "v"(y));
    } else if constexpr (DT == DT_F16) {
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(x), "v"(y));
    } else {
        static_assert(DT == DT_I8, "16x16 blocks: int8, fp16, bf16");
        asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c) : "v"(x), "v"(y));
    }
    return c;
}

// One 32x32 MFMA block step: acc += X * Y over the k values held in one
// 16-byte chunk per lane of each operand.
template <int DT>
__device__ __forceinline__ typename AccT<DT>::type mfma_chunk(i32x4 x, i32x4 y, typename AccT<DT>::type c) {
    if constexpr (DT == DT_BF16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x),
                                                       __builtin_bit_cast(bf16x8, y), c, 0, 0, 0);
    } else if constexpr (DT == DT_F16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, x),
                                                      __builtin_bit_cast(f16x8, y), c, 0, 0, 0);
    } else if constexpr (DT == DT_I8) {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(x, y, c, 0, 0, 0);
    } else {
        // fp32: k = 2 per instruction, element s of each lane's chunk.  (Whole
        // vectors are bit-cast, then indexed: a bit-cast of one vector
        // element would read element 0.)
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 xf = __builtin_bit_cast(f32x4, x), yf = __builtin_bit_cast(f32x4, y);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(xf[0], yf[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(xf[1], yf[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(xf[2], yf[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(xf[3], yf[3], c, 0, 0, 0);
        return c;
    }
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] bits 3:0, expcnt bits
// 6:4, lgkmcnt bits 11:8, vmcnt[5:4] bits 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}

// Every global load and LDS access of this wave has completed.  After the
// direct variant's K loop: no LDS-DMA write may outlive the loop, and the
// last hand-over's fragment reads (in layout RR inline assembly, which the
// compiler does not track) must land before their registers are reused.
__device__ __forceinline__ void wait_all() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((0) | (0 << 14) | (7 << 4) | (0 << 8));
    asm volatile("" ::: "memory");
}

// Workgroup barrier that also drains this wave's LDS accesses first.
__device__ __forceinline__ void block_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int DT, int LAYOUT, int TC, int STAGES, int VARIANT>
struct Gemm {
    static constexpr TileShape TS = tile_shape(TC);
    static constexpr int BM = TS.bm, BN = TS.bn, WM = TS.wm, WN = TS.wn, WK = TS.wk;
    static constexpr int T = WM * WN * WK * 64;
    static constexpr int SZ = in_size(DT), OSZ = out_size(DT), EPC = epc(DT);
    static constexpr int CPR = cpr_k(TC, STAGES, VARIANT); // chunks per K-contiguous row
    static constexpr int BK = CPR * EPC;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    // 16x16 MFMA blocks (see mfma_block16: the 4-wave 256x256 tile's 2-3
    // stage direct rings with K-contiguous B, which carry the large square
    // shapes; two 16x16 steps per K-tile); 32x32 blocks everywhere else.
    static constexpr bool B16 = mfma_block16(DT, LAYOUT, TC, STAGES, VARIANT);
    static constexpr int BS = B16 ? 16 : 32;                // MFMA block edge
    static constexpr int FM = WTM / BS, FN = WTN / BS;
    // MFMA steps of a K-tile per wave (chunks per step: 2 for 32x32 blocks, 4
    // for 16x16); with WK k groups, group g takes steps g KSTEPS .. +KSTEPS-1
    // of the K-tile's CPR / 2.
    static constexpr int KSTEPS = CPR / (B16 ? 4 : 2) / WK;
    static constexpr int LA = loads_a(DT, TC, STAGES, VARIANT), LB = loads_b(DT, TC, STAGES, VARIANT);
    static constexpr int LPT = LA + LB;
    static constexpr int A_BYTES = BM * CPR * kChunk;
    static constexpr int B_BYTES = BN * BK * SZ;
    static constexpr int SLOT = A_BYTES + B_BYTES;
    static constexpr int SLOTS = lds_slots(VARIANT, STAGES);
    static constexpr int RSETS = reg_sets(VARIANT, STAGES);
    static constexpr int LDS = lds_bytes(DT, TC, STAGES, VARIANT);   // the ring, or the epilogue strips
    static constexpr bool RR = (LAYOUT == LAYOUT_RR);
    static constexpr bool SPLIT = split_ring(TC, STAGES, VARIANT);   // three A slots, two B slots
    static constexpr int CPR_BRR = BN * SZ / kChunk;       // chunks per row of a K x N B tile
    static constexpr int RB_RR = BN * SZ;                   // bytes per row of a K x N B tile
    typedef typename std::conditional<B16, i32x4, typename AccT<DT>::type>::type acc_t;

    static_assert(instance_fits(DT, TC, STAGES, VARIANT), "instance over budget");
    static_assert(FM >= 1 && FN >= 1, "wave tile");
    static_assert(T % CPR == 0, "loader rows");
    static_assert(!RR || (BK * CPR_BRR) % T == 0, "RR loader");
    static_assert(LPT * (STAGES > 1 ? STAGES - 1 : 1) < 64, "vmcnt range");
    static_assert(KSTEPS >= 2, "at least two MFMA steps per K-tile");
    static_assert(!B16 || (FM == 8 && FN == 8 && KSTEPS == 2), "16x16 blocks: 8 x 8 per wave, two steps");
    static_assert(WK == 1 || (!B16 && (CPR / 2) % WK == 0), "k groups: 32x32 blocks, whole steps per group");

    // ---- per-lane state --------------------------------------------------
    struct State {
        __amdgpu_buffer_rsrc_t ra, rb;
        uint32_t offa[LA], offb[LB];   // byte offsets at K-tile 0 (rows past M or N: the tile's row 0)
        uint32_t kca[LA], kcb[LB];     // K index the chunk starts at, inside the tile
        uint32_t rd[KSTEPS];           // per-lane LDS read offset of each MFMA step
        uint32_t rd16[B16 ? KSTEPS : 1][2];   // 16x16: the same, per 16-row half of a 32-row group
        uint32_t rrb[RR ? FN : 1];     // layout RR: per-lane B fragment read offset (step 0)
        uint32_t kb_step;              // byte advance of the B offset per K-tile
        int K, nt;                     // K; K-tiles this workgroup multiplies
        int head;                      // K-tiles of the ragged head (0, 1 or 2)
        int nbody, rot;                // the other K-tiles; the one they start at
        int tbase, tail0;              // physical K-tile of body tile 0; of head tile 0
        uint32_t klast;                // K index the last physical K-tile starts at
        int tid, wave, wm, wn, wk;   // wk: the wave's k group (WK > 1)
    };

    __device__ static __forceinline__ void lds_dma(const State& s, bool is_a, uint8_t PG_LDS* dst, uint32_t voff,
                                                   uint32_t soff) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? s.ra : s.rb, (void PG_LDS*)dst, 16, voff, soff, 0, 0);
    }

    // K-tile order (k_phys_tile): the ragged head first, then the rest from
    // `rot`.  The head is defined by BKMAX rather than BK so that instances
    // with BK = BKMAX / 2 add the same k-slices in the same order, and every
    // (stages, variant) pair gives bit-identical C.
    // Register-staged instances compute it with masks: written as
    // conditionals, the compiler made branches of them that split the main
    // loop's scheduled steps, and its waits at the joins cost up to 20%.  The
    // direct instances keep the conditionals: with masks the compiler copied
    // the loop-carried fragments in the 3-4 stage 256x256 loops (16 moves
    // per K-tile, 6% slower), which it does not do with these.  Both forms
    // compute the same tile.
    __device__ static __forceinline__ int phys_tile(const State& s, int t) {
        if constexpr (VARIANT == VAR_DIRECT) {
            return t < s.head ? s.tail0 + t : s.tbase + k_phys_tile(t, s.head, s.nbody, s.rot);
        } else {
            const int b = t - s.head + s.rot;                                // body position, before the wrap
            const int body = s.tbase + b - (s.nbody & -(int)(b >= s.nbody)); // = tbase + k_phys_tile(...)
            const int in_head = -(int)(t < s.head);
            return ((s.tail0 + t) & in_head) | (body & ~in_head);
        }
    }
    // Scalar (wave-uniform) byte offset of logical K-tile t; past the last
    // tile, an offset that takes every lane out of the buffer's range.
    // (readfirstlane states what is true -- every lane holds the same value
    // -- so that the compiler keeps the offset in a scalar register instead
    // of looping over lanes.)
    __device__ static __forceinline__ uint32_t soff_a(const State& s, int t) {
        if constexpr (VARIANT == VAR_DIRECT)
            return __builtin_amdgcn_readfirstlane(t < s.nt ? (uint32_t)phys_tile(s, t) * (uint32_t)(BK * SZ) : kOob);
        const uint32_t past = kOob & (uint32_t)-(int)(t >= s.nt);
        return __builtin_amdgcn_readfirstlane(((uint32_t)phys_tile(s, t) * (uint32_t)(BK * SZ)) | past);
    }
    __device__ static __forceinline__ uint32_t soff_b(const State& s, int t) {
        if constexpr (VARIANT == VAR_DIRECT)
            return __builtin_amdgcn_readfirstlane(t < s.nt ? (uint32_t)phys_tile(s, t) * s.kb_step : kOob);
        const uint32_t past = kOob & (uint32_t)-(int)(t >= s.nt);
        return __builtin_amdgcn_readfirstlane(((uint32_t)phys_tile(s, t) * s.kb_step) | past);
    }
    // Per-lane offset of chunk j.  FIRST: the chunk belongs to the last
    // physical K-tile (logical tile head-1), which may be ragged; chunks
    // starting at or past K move out of range.
    template <bool FIRST>
    __device__ static __forceinline__ uint32_t voff_a(const State& s, int j) {
        if (FIRST && s.kca[j] + s.klast >= (uint32_t)s.K) return kOob;
        return s.offa[j];
    }
    template <bool FIRST>
    __device__ static __forceinline__ uint32_t voff_b(const State& s, int j) {
        if (FIRST && s.kcb[j] + s.klast >= (uint32_t)s.K) return kOob;
        return s.offb[j];
    }

    // DIRECT: issue chunks J0 .. J1-1 of K-tile kt into LDS slot `slot`
    // (chunks 0 .. LA-1 are the A tile, LA .. LPT-1 the B tile).  Chunk j of
    // wave w lands at physical chunk j*T + 64*w + lane, the order LDS-DMA
    // writes in; the lane's source chunk is the logical one stored there.
    template <int J0, int J1, bool FIRST = false>
    __device__ static __forceinline__ void issue_direct(const State& s, uint8_t PG_LDS* smem, int kt, int slot) {
        uint8_t PG_LDS* abase = smem + a_off(slot);
        uint8_t PG_LDS* bbase = smem + b_off(slot);
        const uint32_t sa = soff_a(s, kt), sb = soff_b(s, kt);
#pragma unroll
        for (int j = J0; j < J1; ++j) {
            if (j < LA)
                lds_dma(s, true, abase + (j * T + 64 * s.wave) * kChunk, voff_a<FIRST>(s, j), sa);
            else
                lds_dma(s, false, bbase + ((j - LA) * T + 64 * s.wave) * kChunk, voff_b<FIRST>(s, j - LA), sb);
        }
    }

    // REG: load chunks J0 .. J1-1 of K-tile kt into a VGPR staging set /
    // store a whole set into a slot.
    template <int J0, int J1, bool FIRST = false>
    __device__ static __forceinline__ void gload(const State& s, i32x4 (&r)[LPT], int kt) {
        const uint32_t sa = soff_a(s, kt), sb = soff_b(s, kt);
        if constexpr (FIRST && VARIANT == VAR_REG_KTAIL) {
            // K is not a multiple of EPC: the chunk holding column K-1 is
            // partly past K.
#pragma unroll
            for (int j = J0; j < J1; ++j) {
                if (j < LA)
                    r[j] = load_k_tail(s, s.ra, s.offa[j], s.kca[j], sa);
                else if constexpr (RR)
                    r[j] = __builtin_amdgcn_raw_buffer_load_b128(s.rb, voff_b<true>(s, j - LA), sb, 0);
                else
                    r[j] = load_k_tail(s, s.rb, s.offb[j - LA], s.kcb[j - LA], sb);
            }
            return;
        }
#pragma unroll
        for (int j = J0; j < J1; ++j) {
            if (j < LA)
                r[j] = __builtin_amdgcn_raw_buffer_load_b128(s.ra, voff_a<FIRST>(s, j), sa, 0);
            else
                r[j] = __builtin_amdgcn_raw_buffer_load_b128(s.rb, voff_b<FIRST>(s, j - LA), sb, 0);
        }
    }

    // One K-contiguous chunk of the last physical K-tile when K is not a
    // multiple of EPC: `rem` of its elements lie before K.  rem <= 0 gives
    // zeros, rem >= EPC the whole chunk.  A partial chunk's vb = rem * SZ
    // bytes are read in pieces of 8, 4, 2 and 1 bytes following the binary
    // digits of vb (a piece that is not there takes the out-of-range offset
    // and reads 0), so no byte past K is read and no read passes the end of
    // the matrix; the bytes after vb stay zero.
    __device__ static __forceinline__ i32x4 load_k_tail(const State& s, __amdgpu_buffer_rsrc_t rs, uint32_t off,
                                                       uint32_t kc, uint32_t soff) {
        int rem = s.K - (int)(kc + s.klast);
        // `rem` is the same for every tile; kept opaque, so the compiler forms
        // the offsets below here instead of hoisting them all out of the tile
        // loop into scalar registers (which then spill).
        asm volatile("" : "+v"(rem));
        const uint32_t vb = (rem > 0 && rem < EPC) ? (uint32_t)(rem * SZ) : 0u;
        i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, rem >= EPC ? off : kOob, soff, 0);
        const i32x2 p8 = __builtin_amdgcn_raw_buffer_load_b64(rs, (vb & 8) ? off : kOob, soff, 0);
        const int p4 = (int)__builtin_amdgcn_raw_buffer_load_b32(rs, (vb & 4) ? off + (vb & 8) : kOob, soff, 0);
        uint32_t t = 0;                                     // the 2- and 1-byte pieces: one dword
        if constexpr (SZ <= 2)
            t = __builtin_amdgcn_raw_buffer_load_b16(rs, (vb & 2) ? off + (vb & 12) : kOob, soff, 0);
        if constexpr (SZ == 1)
            t |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, (vb & 1) ? off + (vb & 14) : kOob, soff, 0)
                 << (8 * (vb & 2));
        const uint32_t d4 = (vb & 8) >> 2, dt = (vb & 12) >> 2;   // dwords the 4-byte piece and `t` land in
        v[0] |= p8[0] | (d4 == 0 ? p4 : 0) | (dt == 0 ? (int)t : 0);
        v[1] |= p8[1] | (dt == 1 ? (int)t : 0);
        v[2] |= (d4 == 2 ? p4 : 0) | (dt == 2 ? (int)t : 0);
        v[3] |= (dt == 3 ? (int)t : 0);
        return v;
    }
    __device__ static __forceinline__ void swrite(const State& s, uint8_t PG_LDS* smem, const i32x4 (&r)[LPT], int slot) {
        i32x4 PG_LDS* base = (i32x4 PG_LDS*)(smem + slot * SLOT);
#pragma unroll
        for (int j = 0; j < LA; ++j) base[j * T + s.tid] = r[j];
#pragma unroll
        for (int j = 0; j < LB; ++j) base[A_BYTES / kChunk + j * T + s.tid] = r[LA + j];
    }

    // Prologue load of all of logical K-tile t, with the per-lane K test
    // when t is the last physical tile (the ragged one, if any).
    __device__ static __forceinline__ void first_direct(const State& s, uint8_t PG_LDS* smem, int t, int slot) {
        if (t == s.head - 1)
            issue_direct<0, LPT, true>(s, smem, t, slot);
        else
            issue_direct<0, LPT>(s, smem, t, slot);
    }
    __device__ static __forceinline__ void first_gload(const State& s, i32x4 (&r)[LPT], int t) {
        if (t == s.head - 1)
            gload<0, LPT, true>(s, r, t);
        else
            gload<0, LPT>(s, r, t);
    }

    // Layout RR B fragment (the tile is BK rows of BN N-contiguous
    // elements).  16-bit and 8-bit types: two transposing reads, each giving
    // the lane 4 (8) consecutive k of its column n; s.rrb[fn] is the lane's
    // byte offset for step 0 and the first read, and the k advance of a step
    // or of the second read is a whole number of rows (the swizzle repeats
    // every rr_rows_per_read rows).  fp32: four single-element reads.
    __device__ static __forceinline__ i32x4 read_b_rr(const State& s, const uint8_t PG_LDS* bt, int fn, int st) {
        if constexpr (SZ == 4) {
            const int lane = s.tid & 63;
            const int n = s.wn * WTN + fn * 32 + (lane & 31), k0 = (2 * (s.wk * KSTEPS + st) + (lane >> 5)) * EPC;
            i32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = *(const int PG_LDS*)(bt + ((k0 + e) * BN + n) * 4);
            return v;
        } else {
            return tr_pair(bt + s.rrb[fn] + st * (2 * EPC) * RB_RR);
        }
    }
    // 16x16 blocks: fragment idx covers columns wn*WTN + 16 idx; 16-lane
    // group g holds k rows 4 st + g chunks in (s.rrb[idx] is the lane's
    // offset for step 0; a step advances 4 chunks of k rows).
    __device__ static __forceinline__ i32x4 read_b_rr16(const State& s, const uint8_t PG_LDS* bt, int idx, int st) {
        return tr_pair(bt + s.rrb[idx] + st * (4 * EPC) * RB_RR);
    }
    // Two transposing reads, rr_rows_per_read k rows apart, at p.
    __device__ static __forceinline__ i32x4 tr_pair(const uint8_t PG_LDS* p) {
        {
            typedef int i32x2v __attribute__((ext_vector_type(2)));
            constexpr int RK = rr_rows_per_read(DT);            // k rows per transposing read
            i32x2v lo, hi;
            if constexpr (VARIANT == VAR_DIRECT) {
                // With LDS-DMA writes in flight the compiler cannot tell that
                // these reads touch another slot, and it would drain every
                // outstanding load (vmcnt(0)) before each of them.  Issued as
                // inline assembly they are invisible to its wait insertion:
                // step() waits for them explicitly (lgkmcnt(0) at the start of
                // the step that uses them).  The compiler's own lgkmcnt waits
                // stay correct, only more conservative, because LDS operations
                // complete in order.
                const uint32_t a = (uint32_t)(uintptr_t)p;
                if constexpr (SZ == 2) {
                    asm volatile("ds_read_b64_tr_b16 %0, %2\n\tds_read_b64_tr_b16 %1, %2 offset:%3"
                                 : "=&v"(lo), "=&v"(hi) : "v"(a), "i"(RK * RB_RR) : "memory");
                } else {
                    asm volatile("ds_read_b64_tr_b8 %0, %2\n\tds_read_b64_tr_b8 %1, %2 offset:%3"
                                 : "=&v"(lo), "=&v"(hi) : "v"(a), "i"(RK * RB_RR) : "memory");
                }
            } else if constexpr (SZ == 2) {
                typedef short s16x4 __attribute__((ext_vector_type(4)));
                lo = __builtin_bit_cast(i32x2v, __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 PG_LDS*)p));
                hi = __builtin_bit_cast(i32x2v, __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 PG_LDS*)(p + RK * RB_RR)));
            } else {
                lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2v PG_LDS*)p);
                hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2v PG_LDS*)(p + RK * RB_RR));
            }
            return i32x4{lo[0], lo[1], hi[0], hi[1]};
        }
    }

    // Operand fragments of one MFMA step: FM A-side and FN B-side chunks.
    struct Frags {
        i32x4 y[FM];
        i32x4 x[FN];
    };

    // Byte offsets of the A and B tiles of ring slot `slot`.  Split ring:
    // `slot` is the K-tile index mod 6; its A tile is in A slot slot % 3
    // (the first 3 * A_BYTES of LDS), its B tile in B slot slot % 2.
    __device__ static __forceinline__ uint32_t a_off(int slot) {
        if constexpr (SPLIT) return (uint32_t)(slot - 3 * (int)(slot >= 3)) * A_BYTES;
        else return (uint32_t)slot * SLOT;
    }
    __device__ static __forceinline__ uint32_t b_off(int slot) {
        if constexpr (SPLIT) return 3u * A_BYTES + (uint32_t)(slot & 1) * B_BYTES;
        else return (uint32_t)slot * SLOT + A_BYTES;
    }

    // ---- the MFMA step schedule -------------------------------------------
    //
    // One step = the FM x FN MFMA blocks of one k-slice.  Each block is a
    // "unit" of the schedule: its MFMA(s), then its share of the next step's
    // fragment reads, then its share of global loads, closed by a scheduling
    // fence so the compiler keeps exactly this order (it still inserts every
    // wait the data dependences need).  Reads go early in the step, so the
    // next step's first MFMAs never wait on LDS; loads are spread evenly, so
    // the address unit's queue never fills and stalls the wave's in-order
    // MFMA issue behind it.
    static constexpr int NU = FM * FN;      // units per step
    static constexpr int NRU = FM + FN;     // fragment reads per step (A-side first)
    static constexpr int HALF = LPT / 2;    // loads issued right after the barrier
    // Where a step forms its loads' scalar offsets: once at its start (the
    // 256x256 classes) or at each load (the others).  Same instructions,
    // placed differently; measured, each placement is the one whose loop
    // the compiler keeps in one piece with the fewest waits: the other cost
    // 13% in the 3-stage 256x256 direct loop (a branch inside it) and 3% in
    // the 32x64 one (a wait before every MFMA).
    static constexpr bool HOIST_SOFF = BM == 256;
    // Body steps carrying loads: the first two, or in a split ring (whose A
    // loads run two K-tiles ahead) all of them, which measured 1% faster on
    // bf16 8192^2 x 8200.
    static constexpr int LSTEPS = SPLIT ? KSTEPS - 1 : (KSTEPS - 1 < 2 ? KSTEPS - 1 : 2);
    static constexpr int rd_lo(int u) { return u * ((NRU + NU - 1) / NU) < NRU ? u * ((NRU + NU - 1) / NU) : NRU; }

    // Fragment read r of step st of the K-tile in `slot`.
    __device__ static __forceinline__ void read_one(const State& s, const uint8_t PG_LDS* smem, int slot,
                                                    int st, int r, Frags& f) {
        const uint8_t PG_LDS* as = smem + a_off(slot);
        const uint8_t PG_LDS* bs = smem + b_off(slot);
        if (r < FM) {
            f.y[r] = *(const i32x4 PG_LDS*)(as + (s.wm * WTM + r * 32) * CPR * kChunk + s.rd[st]);
        } else {
            const int fn = r - FM;
            if constexpr (RR)
                f.x[fn] = read_b_rr(s, bs, fn, st);
            else
                f.x[fn] = *(const i32x4 PG_LDS*)(bs + (s.wn * WTN + fn * 32) * CPR * kChunk + s.rd[st]);
        }
    }

    // Load chunk j of logical K-tile kt (never a head tile: those are all
    // loaded in the prologue): into LDS slot `slot` (DIRECT) or regs[j] (REG).
    // sa / sb: the K-tile's scalar offsets when the caller computed them
    // (HOIST_SOFF), else computed here.
    __device__ static __forceinline__ void load_one(const State& s, uint8_t PG_LDS* smem, int kt, uint32_t sa,
                                                    uint32_t sb, int slot, i32x4 (&regs)[LPT], int j) {
        if constexpr (!HOIST_SOFF) {
            sa = soff_a(s, kt);
            sb = soff_b(s, kt);
        }
        if constexpr (VARIANT == VAR_DIRECT) {
            if (j < LA)
                lds_dma(s, true, smem + a_off(slot) + (j * T + 64 * s.wave) * kChunk, s.offa[j], sa);
            else
                lds_dma(s, false, smem + b_off(slot) + ((j - LA) * T + 64 * s.wave) * kChunk, s.offb[j - LA], sb);
        } else {
            if (j < LA)
                regs[j] = __builtin_amdgcn_raw_buffer_load_b128(s.ra, s.offa[j], sa, 0);
            else
                regs[j] = __builtin_amdgcn_raw_buffer_load_b128(s.rb, s.offb[j - LA], sb, 0);
        }
    }

    // One step: MFMAs on `cur`; if RD, read step rd_st of rd_slot into `nxt`;
    // load chunks [J0, J1) of tile ld_kt.  (Called with constant arguments and
    // fully unrolled: every index below is a constant, so fragments and
    // accumulators stay in registers.)
    template <bool RD>
    __device__ static __forceinline__ void step(const State& s, uint8_t PG_LDS* smem, const Frags& cur,
                                                Frags& nxt, int rd_slot, int rd_st, acc_t (&acc)[FM][FN],
                                                int J0, int J1, int ld_kt, int ld_slot, i32x4 (&regs)[LPT]) {
        const int NL = J1 - J0;
        uint32_t ld_sa = 0, ld_sb = 0;
        if constexpr (HOIST_SOFF) {
            if (NL > 0) {
                ld_sa = soff_a(s, ld_kt);
                ld_sb = soff_b(s, ld_kt);
            }
        }
        if constexpr (RR && SZ != 4 && VARIANT == VAR_DIRECT) {
            // the transposing reads of `cur` (inline assembly) have landed
            __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
        }
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int fm = u / FN, fn = u % FN;
            acc[fm][fn] = mfma_chunk<DT>(cur.x[fn], cur.y[fm], acc[fm][fn]);
            if constexpr (RD) {
#pragma unroll
                for (int r = rd_lo(u); r < rd_lo(u + 1); ++r) read_one(s, smem, rd_slot, rd_st, r, nxt);
            }
#pragma unroll
            for (int j = J0 + u * NL / NU; j < J0 + (u + 1) * NL / NU; ++j)
                load_one(s, smem, ld_kt, ld_sa, ld_sb, ld_slot, regs, j);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ---- 16x16 blocks (B16) -------------------------------------------------
    //
    // A wave's 128x128 block is 8 x 8 blocks of 16x16, and a step (4 chunks
    // of k) needs 8 A-side and 8 B-side fragments -- twice the 32x32 step's.
    // Double-buffered they would not fit the 256 arch VGPRs, so there is one
    // fragment set, refilled in quadrant order: a step runs quadrants
    // (A 0-3 x B 0-3), (A 0-3 x B 4-7), (A 4-7 x B 0-3), (A 4-7 x B 4-7).
    // It reads its own fragments B 4-7 and A 4-7 during the first quadrant,
    // the next step's A 0-3 during the third (their last use was the second)
    // and the next step's B 0-3 during the fourth (last use: the third).
    // Every read has 4-12 MFMAs between the last use of its registers and
    // itself, and 12 or more before its first use.
    //
    // Fragment idx of a side (0-7: rows 16 idx .. of the wave's block) of
    // step st of the K-tile in `slot`: lane l takes row (l % 16) and chunk
    // (4 st + l / 16).
    __device__ static __forceinline__ void read16(const State& s, const uint8_t PG_LDS* smem, int slot, int st,
                                                  bool a_side, int idx, Frags& f) {
        if (a_side)
            f.y[idx] = *(const i32x4 PG_LDS*)(smem + a_off(slot) + (s.wm * WTM + (idx >> 1) * 32) * CPR * kChunk +
                                              s.rd16[st][idx & 1]);
        else if constexpr (RR)
            f.x[idx] = read_b_rr16(s, smem + b_off(slot), idx, st);
        else
            f.x[idx] = *(const i32x4 PG_LDS*)(smem + b_off(slot) + (s.wn * WTN + (idx >> 1) * 32) * CPR * kChunk +
                                              s.rd16[st][idx & 1]);
    }
    // One 16x16 step: MFMAs on the fragments of step cst of `cslot` (A/B
    // 0-3 already in f), reading the rest and the next step's (nslot, nst)
    // A/B 0-3 as above; loads of chunks [J0, J1) of K-tile ld_kt.  BAR: the
    // hand-over to the next K-tile -- wait for its data and cross the barrier
    // after the first (split ring) or second quadrant, once this step's own
    // reads of its slot have completed (the barrier frees the slot for the
    // loads that follow), and issue the loads after it.
    template <bool BAR, int WAITN>
    __device__ static __forceinline__ void step16(const State& s, uint8_t PG_LDS* smem, Frags& f, int cslot,
                                                  int cst, int nslot, int nst, acc_t (&acc)[FM][FN], int J0,
                                                  int J1, int ld_kt, int ld_slot, i32x4 (&regs)[LPT]) {
        const int NL = J1 - J0;
        // The hand-over's wait and barrier: after the first quadrant in the
        // split ring, after the second otherwise (the 2-stage ring's wait for
        // the next tile then comes 16 MFMAs later; measured 3-6% faster at
        // 2 stages, no change in the split ring).  Either way this step's own
        // reads of its slot (first quadrant) are done and the next step's
        // reads (third and fourth) come after it.
        constexpr int BAR_U = SPLIT ? 15 : 31;
        constexpr int LU0 = BAR ? BAR_U + 1 : 0;     // loads go in units [LU0, 64)
        uint32_t ld_sa = 0, ld_sb = 0;
#pragma unroll
        for (int u = 0; u < 64; ++u) {
            const int q = u / 16, i = u % 16;
            const int fm = (q >> 1) * 4 + i / 4, fn = (q & 1) * 4 + i % 4;
            if constexpr (RR && VARIANT == VAR_DIRECT) {
                // Layout RR's B reads are inline assembly (see tr_pair), so
                // their waits are explicit: B 0-3 (read in the previous step)
                // before the first quadrant; B 4-7 (read in the first
                // quadrant, followed by exactly the 4 reads of A 4-7) before
                // the second.  LDS reads complete in order.
                if (u == 0) __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
                if (u == 16) __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (4 << 8));
            }
            acc[fm][fn] = mfma16<DT>(f.x[fn], f.y[fm], acc[fm][fn]);
            if (q == 0 && (i & 1) == 0) {
                const int r = i / 2;                  // B 4-7, then A 4-7
                read16(s, smem, cslot, cst, r >= 4, 4 + (r & 3), f);
            }
            if (q == 2 && (i & 3) == 0) read16(s, smem, nslot, nst, true, i / 4, f);
            if (q == 3 && i < 4) read16(s, smem, nslot, nst, false, i, f);
            if (u >= LU0) {
                if (u == LU0 && NL > 0) {
                    ld_sa = soff_a(s, ld_kt);
                    ld_sb = soff_b(s, ld_kt);
                }
#pragma unroll
                for (int j = J0 + (u - LU0) * NL / (64 - LU0); j < J0 + (u - LU0 + 1) * NL / (64 - LU0); ++j)
                    load_one(s, smem, ld_kt, ld_sa, ld_sb, ld_slot, regs, j);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (BAR && u == BAR_U) {
                wait_vmcnt<WAITN>();
                block_sync();
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    // The MFMAs above are inline assembly, so the compiler inserts none of
    // the wait states around them.  Each K-tile starts with a few (the
    // accumulators' initial values are ordinary moves made just before the
    // loop), and the loop is followed by more than any MFMA result needs
    // before the epilogue reads the accumulators.  (Tying the accumulators
    // to the padding with empty statements instead made the compiler spill
    // 53 VGPRs outside the loop.)
    __device__ static __forceinline__ void mfma16_pad_tile() { asm volatile("s_nop 4" ::: "memory"); }
    __device__ static __forceinline__ void mfma16_pad_after() {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    }

    // Steps 0 .. KSTEPS-2 of the K-tile in `slot`.  On entry f[0] holds step
    // 0's fragments; each step reads the next step's while its MFMAs run (a
    // two-deep register pipeline).  When LOADS, the first LSTEPS steps also
    // carry chunks [HALF, LPT) of K-tile ld_kt (the chunks [0, HALF) went out
    // right after the previous barrier); in a split ring, its A chunks
    // [0, LA) (its B chunks follow the next barrier).  KSTEPS is even, so on
    // exit f[1] holds the last step's fragments and f[0] is free for the next
    // tile.
    template <bool LOADS>
    __device__ static __forceinline__ void tile_body(const State& s, uint8_t PG_LDS* smem, int slot,
                                                     Frags (&f)[2], acc_t (&acc)[FM][FN], int ld_kt,
                                                     int ld_slot, i32x4 (&regs)[LPT]) {
        static_assert(KSTEPS % 2 == 0, "step parity");
        constexpr int BJ0 = SPLIT ? 0 : HALF, BJ1 = SPLIT ? LA : LPT;   // chunks the body carries
        constexpr int REST = BJ1 - BJ0;
#pragma unroll
        for (int st = 0; st + 1 < KSTEPS; ++st) {
            const int j0 = (LOADS && st < LSTEPS) ? BJ0 + st * REST / LSTEPS : 0;
            const int j1 = (LOADS && st < LSTEPS) ? BJ0 + (st + 1) * REST / LSTEPS : 0;
            step<true>(s, smem, f[st & 1], f[(st + 1) & 1], slot, st + 1, acc, j0, j1, ld_kt, ld_slot, regs);
        }
    }

    // Read every fragment of step 0 of `slot` into f (no MFMA to overlap).
    __device__ static __forceinline__ void read_first(const State& s, const uint8_t PG_LDS* smem, int slot, Frags& f) {
#pragma unroll
        for (int r = 0; r < NRU; ++r) read_one(s, smem, slot, 0, r, f);
    }

    // One K-tile of the register-staged ring with R staging sets: tile kt
    // travels in set i = kt % R; while it is multiplied, tile kt+R is loaded
    // into set i, which tile kt has just left.
    template <int R>
    __device__ static __forceinline__ void reg_tile(const State& s, uint8_t PG_LDS* smem, Frags (&f)[2],
                                                    acc_t (&acc)[FM][FN], i32x4 (&regs)[RSETS][LPT], int kt,
                                                    int i) {
        tile_body<true>(s, smem, kt & 1, f, acc, kt + R, 0, regs[i]);
        // buffer (kt+1)&1 was last read in iteration kt-1, before that
        // iteration's barrier
        swrite(s, smem, regs[(i + 1) % R], (kt + 1) & 1);
        block_sync();
        step<true>(s, smem, f[1], f[0], (kt + 1) & 1, 0, acc, 0, HALF, kt + 1 + R, 0, regs[(i + 1) % R]);
    }

    // WK > 1: add the k groups' partial accumulators into group 0.  Groups
    // 1 .. WK-1 store theirs in LDS (block, quarter, lane order, so 8
    // consecutive lanes write 128 contiguous bytes: no bank conflict), and
    // group 0 adds them in group order.  The ring is free: every wave's
    // loads into LDS have completed (direct variant) and the barrier drains
    // its LDS reads.
    __device__ static __forceinline__ void add_k_groups(const State& s, uint8_t PG_LDS* smem, acc_t (&acc)[FM][FN]) {
        constexpr int WB = FM * FN * 4 * 64 * 16;       // bytes per wave
        static_assert((WK - 1) * WM * WN * WB <= LDS, "k-group sums fit the LDS");
        const int lane = s.tid & 63, wmn = s.wave % (WM * WN);
        block_sync();
        if (s.wk > 0) {
            uint8_t PG_LDS* base = smem + ((s.wk - 1) * WM * WN + wmn) * WB;
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *(i32x4 PG_LDS*)(base + (((fm * FN + fn) * 4 + q) * 64 + lane) * 16) = out4_32(acc[fm][fn], q);
        }
        block_sync();
        if (s.wk == 0) {
#pragma unroll
            for (int g = 1; g < WK; ++g) {
                const uint8_t PG_LDS* base = smem + ((g - 1) * WM * WN + wmn) * WB;
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const i32x4 v = *(const i32x4 PG_LDS*)(base + (((fm * FN + fn) * 4 + q) * 64 + lane) * 16);
                            const f32x4 vf = __builtin_bit_cast(f32x4, v);   // whole vector, then index
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                if constexpr (DT == DT_I8)
                                    acc[fm][fn][4 * q + e] += v[e];
                                else
                                    acc[fm][fn][4 * q + e] += vf[e];
                            }
                        }
            }
        }
    }

    // Partial tiles (split K, stream-K).  Each contributor of a tile writes
    // its accumulators to the workspace as a BM x BN tile of 4-byte words
    // and counts itself in the tile's arrival counter.  The contributor that
    // arrives last adds the partial tiles in K order, rounds once and
    // stores C; the others are done.  Nothing waits for another workgroup,
    // and the sum's order does not depend on which contributor is last.  The
    // last one puts the counter back to 0, so the counters are zero again
    // after every call.
    //   Split K (mode 1): contributor p of `splits` writes slot p of the
    // tile's own `splits` slots.  Stream-K (mode 2): the contributors of
    // tile t are the workgroups sk_owner(first unit) .. sk_owner(last unit),
    // each writing the slot sk_slot gives it (slot `part`).
    //   Visibility across XCDs (each has its own L2) without an L2-wide
    // write-back or invalidate: the partials are written and read with
    // device-scope stores and loads (the scope bits of the buffer
    // instructions: written through to memory, read from it), every store
    // has completed before the counter is incremented, and the partials are
    // read only after the increment that finds all the others.
    //   workspace: kSplitkCounters uint32 counters, then the partial tiles:
    //   split K [ntiles][splits][BM][BN], stream-K [2 x grid][BM][BN] words.
    __device__ static __forceinline__ void partial(const GemmArgs& args, uint8_t PG_LDS* smem, const State& s,
                                                   const acc_t (&acc)[FM][FN], int mode, int part, int j, int m0,
                                                   int n0) {
        constexpr int PART = BM * BN * 4;
        const int tile = (m0 / BM) * args.tiles_n + n0 / BN;   // any one-to-one tile number will do
        uint32_t* cnt = (uint32_t*)args.ws;
        uint8_t* tp = (uint8_t*)args.ws + kSplitkCounterBytes + (mode == 1 ? (size_t)tile * args.splits * PART : 0);
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(tp, 0, 0x7fffffff, kRsrcWord3);
        // Contributors of the tile, and the first one's stream-K numbers.
        constexpr int BKMAX = block_k(DT, TC, 1, VARIANT);
        const int64_t U = args.K / BKMAX > 0 ? args.K / BKMAX : 1, G = gridDim.x;
        const int64_t total = (int64_t)args.sk_tiles * U;
        const int64_t t0 = (int64_t)(j - (args.tiles_m * args.tiles_n - args.sk_tiles)) * U;
        const int64_t g0 = mode == 2 ? sk_owner(t0, G, total) : 0;
        const int nparts = mode == 2 ? (int)(sk_owner(t0 + U - 1, G, total) - g0 + 1) : args.splits;
        // 1. Lane (t, h) holds row t, columns 8q + 4h .. +3 of each 32x32 block
        //    (per-lane offset in the vector operand, the block's in the scalar
        //    one); 16x16 blocks likewise.  With k groups, group 0 holds the
        //    sums.
        if (WK > 1 && s.wk != 0) {
            // no partial of its own
        } else if constexpr (B16) {
            // 16x16 blocks: lane l holds row (l % 16), columns 4 (l / 16) .. +3
            const int lane = s.tid & 63;
            const uint32_t vo = (uint32_t)(((s.wm * WTM + (lane & 15)) * BN + s.wn * WTN + 4 * (lane >> 4)) * 4);
            const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)part * PART);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    __builtin_amdgcn_raw_buffer_store_b128(acc[fm][fn], rw, vo,
                                                           so + (uint32_t)((fm * 16 * BN + fn * 16) * 4), kScopeDevice);
        } else {
            const int lane = s.tid & 63, t = lane & 31, h = lane >> 5;
            const uint32_t vo = (uint32_t)(((s.wm * WTM + t) * BN + s.wn * WTN + 4 * h) * 4);
            const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)part * PART);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        __builtin_amdgcn_raw_buffer_store_b128(out4_32(acc[fm][fn], q), rw, vo,
                                                               so + (uint32_t)((fm * 32 * BN + fn * 32 + 8 * q) * 4),
                                                               kScopeDevice);
        }
        wait_vmcnt<0>();                   // this workgroup's partial has reached memory ...
        block_sync();
        if (s.tid == 0)                    // ... before it is counted
            *(volatile uint32_t PG_LDS*)smem =
                __hip_atomic_fetch_add(&cnt[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (uint32_t)(nparts - 1);
        block_sync();
        if (*(volatile uint32_t PG_LDS*)smem == 0) return;
        // 2. Four consecutive columns per lane and iteration (a wave covers
        //    256 contiguous words of the tile per iteration), in chunks of CH
        //    iterations: a contributor's CH loads of a chunk are in flight
        //    together, and the next contributor's are issued before the
        //    current one's are added, so a chunk costs about one memory
        //    latency instead of one per iteration and contributor (summing
        //    one 16-byte word at a time made the finisher of a 256x256 tile
        //    latency-bound: 64 iterations x contributors round trips).
        //    Contributors are added in K order.
        //    Only the 4-wave 256x256 tile batches iterations (CH = 8): it
        //    runs one wave per SIMD with registers to spare, while in the
        //    other classes the chunk's 3 x CH x 4 registers raised the
        //    kernel's register peak (fewer waves per SIMD, or spills in the
        //    8-wave tile).
        constexpr int ITER = BM * BN / (4 * T);
        constexpr int CH = TC == TILE_L ? 8 : 1;
        static_assert(ITER % CH == 0, "finisher chunks");
        for (int it0 = 0; it0 < ITER; it0 += CH) {
            i32x4 sum[CH], cur[CH], nxt[CH];
            auto fetch = [&](i32x4 (&v)[CH], int q) {
                const int slot = mode == 2 ? (int)sk_slot(g0 + q, t0, G, total) : q;
                const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)slot * PART);
#pragma unroll
                for (int u = 0; u < CH; ++u)
                    v[u] = __builtin_amdgcn_raw_buffer_load_b128(rw, (uint32_t)(((it0 + u) * T + s.tid) * 16), so,
                                                                 kScopeDevice);
            };
#pragma unroll
            for (int u = 0; u < CH; ++u) sum[u] = i32x4{0, 0, 0, 0};
            fetch(cur, 0);
            for (int q = 0; q + 1 < nparts; ++q) {
                fetch(nxt, q + 1);
#pragma unroll
                for (int u = 0; u < CH; ++u) {
                    sum[u] = add_acc(sum[u], cur[u]);
                    cur[u] = nxt[u];
                }
            }
#pragma unroll
            for (int u = 0; u < CH; ++u) {
                sum[u] = add_acc(sum[u], cur[u]);
                const int idx = ((it0 + u) * T + s.tid) * 4;
                const int m = idx / BN, n = idx % BN;
                if (m0 + m < args.M) store_out4(args, m0 + m, n0 + n, sum[u]);
            }
        }
        if (s.tid == 0) __hip_atomic_store(&cnt[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // A workgroup's work: the data-parallel tiles blockIdx.x, blockIdx.x +
    // gridDim.x, ... (with K split in `splits` parts, work item j is split
    // j / ntiles of tile j % ntiles: consecutive workgroups share a K range);
    // then, when the last sk_tiles tiles are shared out stream-K, its range
    // of their units (sk_begin), one piece per tile it touches.
    __device__ static __forceinline__ void run(const GemmArgs args, uint8_t PG_LDS* smem) {
        constexpr int BKMAX = block_k(DT, TC, 1, VARIANT);
        const int units = args.K / BKMAX;
        const int ndp = args.tiles_m * args.tiles_n - args.sk_tiles;
        const int nwork = ndp * args.splits;
        const int64_t U = units > 0 ? units : 1;   // stream-K: a K below one unit is one unit, the head
        const int64_t G = gridDim.x, total = (int64_t)args.sk_tiles * U;
        // Stream-K calls number the workgroups XCD by XCD (workgroup b runs
        // on XCD b mod 8), so that the workgroups of one XCD take
        // consecutive data-parallel tiles and a consecutive run of units,
        // and take the tiles in plain band order: the tiles an XCD works on
        // at a time then share A rows and B columns in its L2, as the
        // regrouping in run_tile arranges for the other calls.
        const bool skm = args.sk_tiles > 0;
        const int vb = (skm && (gridDim.x & 7) == 0) ? (int)((blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3))
                                                     : (int)blockIdx.x;
        const int64_t i0 = skm ? sk_begin(vb, G, total) : 0;
        const int64_t e = skm ? sk_begin(vb + 1, G, total) : 0;
        int64_t i = i0;
        bool first = true;
        // One call site of run_tile (it is inlined): each pass takes the
        // next data-parallel item, else the next stream-K piece.
        for (int j = vb;;) {
            int tile, u0, u1, mode, part, rot_u = -1;
            bool last;
            if (j < nwork) {
                const int p = j / ndp;
                tile = j - p * ndp;
                u0 = p * units / args.splits;
                u1 = (p + 1) * units / args.splits;
                last = p == args.splits - 1;
                mode = args.splits > 1 ? 1 : 0;
                part = p;
                j += gridDim.x;
            } else if (i < e) {
                const int64_t t = i / U, a = i - t * U, b = sk_piece_end(i, e, U);
                tile = ndp + (int)t;
                u0 = (int)(a < units ? a : units);
                u1 = (int)(b < units ? b : units);
                last = b == U;
                mode = (a == 0 && b == U) ? 0 : 2;
                part = (int)(2 * vb + (i == i0 ? 0 : 1));
                // Keep the workgroups of an XCD on one K unit at a time, as
                // in the data-parallel rounds (unit 9x + step of XCD x; the
                // workgroups of an XCD work on neighbouring tiles, which
                // then share A rows and B columns in its L2 only if they
                // read the same K columns together): start the piece at the
                // unit that puts this workgroup's step i - i0 on that unit,
                // or, when that unit lies outside the piece, at the unit
                // that reaches it when it enters.
                const int64_t len = b - a, d = (i - i0 + 9 * (int64_t)(blockIdx.x & 7) + U - a % U) % U;
                rot_u = (int)((((d >= len ? d - U : d) % len) + len) % len);
                i += b - a;
            } else {
                break;
            }
            if (!first) block_sync();   // every wave is done with the last strips
            first = false;
            run_tile(args, smem, tile, u0, u1, last, mode, part, skm, rot_u);
        }
    }

    // Tile j, units [u0, u1) of its K loop (the ragged head too when
    // `last`); mode 0 stores C, mode 1 writes split `part`'s partial tile,
    // mode 2 stream-K partial slot `part` (summed by whichever contributor
    // of the tile arrives last).  The K loop starts at unit u0 + rot_u
    // (rot_u >= 0) or at the XCD's rotation (rot_u = -1).
    __device__ static __forceinline__ void run_tile(const GemmArgs args, uint8_t PG_LDS* smem, int j, int u0,
                                                    int u1, bool last, int mode, int part, bool band_order,
                                                    int rot_u) {
        const int ntiles = args.tiles_m * args.tiles_n;
        State s;
        s.tid = threadIdx.x;
        s.wave = __builtin_amdgcn_readfirstlane(s.tid >> 6);
        s.wk = s.wave / (WM * WN);
        s.wm = (s.wave % (WM * WN)) / WN;
        s.wn = s.wave % WN;
        const int lane = s.tid & 63;

        // Tile index -> C tile.  Workgroups are handed to the 8 XCDs round
        // robin, so tile j runs on XCD j % 8 (the grid is a multiple of 8);
        // regroup so that each XCD gets a contiguous run of tiles, and order
        // the runs in bands of kGroupM tile-rows so that the tiles one XCD
        // holds at a time share A rows and B columns in its L2.  (With
        // band_order the caller has numbered the tiles that way already.)
        int w = j;
        if (!band_order && (ntiles & 7) == 0 && (gridDim.x & 7) == 0) w = (w & 7) * (ntiles >> 3) + (w >> 3);
        constexpr int kGroupM = 4;
        const int band = kGroupM * args.tiles_n;
        const int g = w / band;
        const int first_m = g * kGroupM;
        const int gm = min(args.tiles_m - first_m, kGroupM);
        const int r_in = w - g * band;
        const int tm = first_m + r_in % gm;
        const int tn = r_in / gm;
        const int m0 = tm * BM, n0 = tn * BN;

        s.K = args.K;
        {
            // K splits and stream-K pieces are whole BKMAX-wide units, so
            // that every stage count adds the same k-slices in the same
            // order; the ragged head goes with the piece that holds the
            // tile's last unit.
            constexpr int BKMAX = block_k(DT, TC, 1, VARIANT);
            static_assert(BKMAX % BK == 0 && (BKMAX == BK || STAGES >= 3), "head tiles are all in the prologue");
            const int head = k_head_tiles(args.K, BK, BKMAX);
            const int units = args.K / BKMAX, per = BKMAX / BK;
            s.head = last ? head : 0;
            s.nbody = (u1 - u0) * per;
            s.nt = s.nbody + s.head;
            s.tbase = u0 * per;
            s.tail0 = units * per;
            s.klast = (uint32_t)(units * per + head - 1) * BK;
            // Start the K loop of the tiles on XCD x at unit 9x (mod the
            // count): with every XCD reading the same K columns at once, the
            // row-strided reads pile onto the same HBM channels (measured on
            // the skinny 8192x64x8192 shape: 4.0 -> 4.5 TB/s; on 8192^2 x
            // 8200 with 256x256 tiles, 3-7% at every stage count).  Within an
            // XCD the tiles keep a common K position, so they still share
            // operands in its L2.  The 256x256 tiles rotate only when the
            // workgroups loop over more work than one pass (operands then
            // stream from HBM): with one tile per CU (4096^3, operands held
            // in the Infinity Cache) XCDs that share A rows gain from
            // reading them together, and rotating cost the 3-4 stage
            // instances 6%.  Counted in BKMAX units, so every stage count
            // starts at the same k-slice; every (stages, variant) pair of a
            // call takes the same decision.
            const bool rotate = BM < 256 || args.tiles_m * args.tiles_n * args.splits > (int)gridDim.x;
            const uint32_t xcd = band_order ? (blockIdx.x & 7) : (uint32_t)(j & 7);
            s.rot = rot_u >= 0 ? rot_u * per
                  : (rotate && u1 > u0) ? (int)((xcd * 9u) % (uint32_t)(u1 - u0)) * per : 0;
        }
        const uint8_t* A = (const uint8_t*)args.A + (int64_t)m0 * args.lda * SZ;
        const uint8_t* B = RR ? (const uint8_t*)args.B + (int64_t)n0 * SZ
                              : (const uint8_t*)args.B + (int64_t)n0 * args.ldb * SZ;
        s.ra = __builtin_amdgcn_make_buffer_rsrc((void*)A, 0, 0x7fffffff, kRsrcWord3);
        s.rb = __builtin_amdgcn_make_buffer_rsrc((void*)B, 0, 0x7fffffff, kRsrcWord3);
        const uint32_t lda_b = (uint32_t)(args.lda * SZ), ldb_b = (uint32_t)(args.ldb * SZ);

#pragma unroll
        for (int j = 0; j < LA; ++j) {
            const int p = j * T + s.tid;
            const int r = logical_row(CPR, p), c = logical_chunk(CPR, p);
            const int rr = (m0 + r < args.M) ? r : 0;
            s.offa[j] = (uint32_t)rr * lda_b + (uint32_t)(c * EPC * SZ);
            s.kca[j] = (uint32_t)(c * EPC);
        }
        if constexpr (RR) {
            // B tile: BK rows (k) of BN elements (n); physical chunk pc of row
            // r holds logical chunk pc ^ swz_rr(r).
#pragma unroll
            for (int j = 0; j < LB; ++j) {
                const int p = j * T + s.tid;
                const int r = p / CPR_BRR, c = (p % CPR_BRR) ^ swz_rr(DT, RB_RR, r);
                const int cc = (n0 + c * EPC < args.N) ? c : 0;
                s.offb[j] = (uint32_t)r * ldb_b + (uint32_t)(cc * EPC * SZ);
                s.kcb[j] = (uint32_t)r;
            }
            s.kb_step = (uint32_t)BK * ldb_b;
            if constexpr (SZ != 4) {
                // Transposing reads: each lane supplies the piece of row k
                // at column n (rr_lane_k / rr_lane_n; 16x16 blocks: group g
                // takes the fragment's 16 columns at its own chunk g of k,
                // the order the K-contiguous read gives).
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    const int k = rr_lane_k(DT, B16, lane);
                    const int n = s.wn * WTN + fn * BS + rr_lane_n(DT, B16, lane);
                    const int c = n * SZ / kChunk, b = n * SZ % kChunk;
                    // (the k group's first step: its k rows start 2 EPC per step on,
                    // a whole number of swizzle periods)
                    s.rrb[fn] = (uint32_t)(k * RB_RR + (c ^ swz_rr(DT, RB_RR, k)) * kChunk + b) +
                                (uint32_t)(s.wk * KSTEPS * 2 * EPC * RB_RR);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < LB; ++j) {
                const int p = j * T + s.tid;
                const int r = logical_row(CPR, p), c = logical_chunk(CPR, p);
                const int rr = (n0 + r < args.N) ? r : 0;
                s.offb[j] = (uint32_t)rr * ldb_b + (uint32_t)(c * EPC * SZ);
                s.kcb[j] = (uint32_t)(c * EPC);
            }
            s.kb_step = (uint32_t)(BK * SZ);
        }
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st) {
            const int t = lane & 31, h = lane >> 5;
            if constexpr (B16) {
                s.rd[st] = 0;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    // the swizzle depends on the row mod 32; fragments start at multiples of 16
                    const int row = 16 * half + (lane & 15), c = 4 * st + (lane >> 4);
                    s.rd16[st][half] = (uint32_t)(row * CPR + (c ^ swz(CPR, row))) * kChunk;
                }
            } else {
                s.rd[st] = (uint32_t)(t * CPR + ((2 * (s.wk * KSTEPS + st) + h) ^ swz(CPR, t))) * kChunk;
            }
        }

        acc_t acc[FM][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int v = 0; v < (B16 ? 4 : 16); ++v) acc[fm][fn][v] = 0;

        // Every loop below is the K-tile loop restructured into prologue /
        // main loop / drain.  Each K-tile runs steps 0..KSTEPS-2 (tile_body);
        // the hand-over to the next tile -- wait for its data, barrier, read
        // its first fragments, start refilling the slot every wave has just
        // finished with -- runs under the last step's MFMAs.  Tiles at or past
        // nt are still loaded: every one of their offsets is out of the
        // buffer's range, so they move no data and only write zeros into a
        // slot (or register set) no later tile reads.  The number of loads in
        // flight is then the same at every boundary, so each wait is a fixed
        // vmcnt and the loop body has no branch.  (The hand-over also runs
        // after the last tile; the fragments it reads are never used.)
        const int nt = s.nt;
        Frags f[2];
        if constexpr (VARIANT == VAR_DIRECT && STAGES == 1) {
            // Unpipelined: load, wait, barrier, compute, barrier.  (The
            // load of tile kt+1 is issued at the end of iteration kt.)
            i32x4 none[LPT];
            first_direct(s, smem, 0, 0);
            for (int kt = 0; kt < nt; ++kt) {
                wait_vmcnt<0>();
                block_sync();
                read_first(s, smem, 0, f[0]);
                tile_body<false>(s, smem, 0, f, acc, 0, 0, none);
                step<false>(s, smem, f[1], f[0], 0, 0, acc, 0, 0, 0, 0, none);
                block_sync();
                issue_direct<0, LPT>(s, smem, kt + 1, 0);
            }
            wait_all();   // no LDS write or fragment read may outlive the loop
        } else if constexpr (VARIANT == VAR_DIRECT) {
            // Ring of STAGES slots: while tile kt is multiplied, tiles
            // kt+1 .. kt+STAGES-1 are in flight; tile kt+STAGES-1 goes into
            // the slot tile kt-1 used.  Split ring (slots counted mod 6):
            // while tile kt is multiplied, the A tile of kt+2 goes into the A
            // slot tile kt-1 used; after the barrier that ends tile kt, the B
            // tile of kt+2 goes into the B slot tile kt used.  At that
            // barrier only the A tile of kt+2 may still be in flight.
            i32x4 none[LPT];
            constexpr int NSLOT = SPLIT ? 6 : STAGES;
            constexpr int WAITN = SPLIT ? LA : (STAGES - 2) * LPT;
            constexpr int HJ0 = SPLIT ? LA : 0, HJ1 = SPLIT ? LPT : HALF, HKT = SPLIT ? 2 : STAGES;
#pragma unroll
            for (int t = 0; t < STAGES - 1; ++t) first_direct(s, smem, t, t);
            wait_vmcnt<(STAGES - 2) * LPT>();
            block_sync();
            if constexpr (B16) {
                // fragments A/B 0-3 of step 0 (the rest are read in its first quadrant)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    read16(s, smem, 0, 0, true, i, f[0]);
                    read16(s, smem, 0, 0, false, i, f[0]);
                }
            } else {
                read_first(s, smem, 0, f[0]);
            }
            if constexpr (!SPLIT) issue_direct<0, HALF>(s, smem, STAGES - 1, STAGES - 1);
            int slot = 0;
            if constexpr (B16) {
                // Step 0 carries the loads the body steps carry below; step
                // 1 is the hand-over.
                constexpr int BJ0 = SPLIT ? 0 : HALF, BJ1 = SPLIT ? LA : LPT;
                for (int kt = 0; kt < nt; ++kt) {
                    const int prev = (slot == 0) ? NSLOT - 1 : slot - 1;
                    const int next = (slot + 1 == NSLOT) ? 0 : slot + 1;
                    mfma16_pad_tile();
                    step16<false, 0>(s, smem, f[0], slot, 0, slot, 1, acc, BJ0, BJ1, kt + STAGES - 1, prev, none);
                    step16<true, WAITN>(s, smem, f[0], slot, 1, next, 0, acc, HJ0, HJ1, kt + HKT, slot, none);
                    slot = next;
                }
                mfma16_pad_after();
            } else {
            for (int kt = 0; kt < nt; ++kt) {
                const int prev = (slot == 0) ? NSLOT - 1 : slot - 1;
                const int next = (slot + 1 == NSLOT) ? 0 : slot + 1;
                tile_body<true>(s, smem, slot, f, acc, kt + STAGES - 1, prev, none);
                wait_vmcnt<WAITN>();                 // tile kt+1 landed (this wave)
                block_sync();                        // ...all waves; slot of kt free
                step<true>(s, smem, f[1], f[0], next, 0, acc, HJ0, HJ1, kt + HKT, slot, none);
                slot = next;
            }
            }
            wait_all();   // no LDS write or fragment read may outlive the loop
        } else {
            i32x4 regs[RSETS][LPT];
            if constexpr (STAGES == 1) {
                // One LDS buffer, one register set: tile kt+1 is loaded into
                // registers while tile kt is multiplied (register prefetch).
                first_gload(s, regs[0], 0);
                swrite(s, smem, regs[0], 0);
                block_sync();
                read_first(s, smem, 0, f[0]);
                gload<0, HALF>(s, regs[0], 1);
                for (int kt = 0; kt < nt; ++kt) {
                    tile_body<true>(s, smem, 0, f, acc, kt + 1, 0, regs[0]);
                    block_sync();                 // every wave done reading the buffer
                    swrite(s, smem, regs[0], 0);  // tile kt+1 (zeros past the end)
                    block_sync();
                    step<true>(s, smem, f[1], f[0], 0, 0, acc, 0, HALF, kt + 2, 0, regs[0]);
                }
            } else {
                // Two LDS buffers, R = STAGES-1 register sets: tile j travels
                // in set j % R; while tile kt is multiplied, tile kt+R is
                // loaded into the set tile kt has just left.
                constexpr int R = RSETS;
#pragma unroll
                for (int t = 0; t < R; ++t) first_gload(s, regs[t], t);
                swrite(s, smem, regs[0], 0);
                block_sync();
                read_first(s, smem, 0, f[0]);
                gload<0, HALF>(s, regs[0], R);
                // Whole groups of R tiles, so that set indices are constants
                // (a guard inside the unrolled group makes the compiler
                // spill).  The up to R-1 tiles past nt hold zeros only: the
                // accumulators start at +0, and adding exact zero products
                // under round-to-nearest leaves every accumulator bit as it
                // was, so C is unchanged.
                for (int kb = 0; kb < nt; kb += R) {
#pragma unroll
                    for (int i = 0; i < R; ++i) reg_tile<R>(s, smem, f, acc, regs, kb + i, i);
                }
            }
        }

        if constexpr (WK > 1) add_k_groups(s, smem, acc);
        if (mode != 0) {
            partial(args, smem, s, acc, mode, part, j, m0, n0);
            return;
        }

        // Epilogue.  Lane (t, h) holds C[m][n .. n+3] of each 32x32 block
        // (m = row t of the block, n = 8q + 4h), so a direct store would
        // scatter 8-16 bytes over 32 rows per instruction.  Instead each
        // wave stages one 32-row strip of its block at a time in a private
        // LDS region and reads it back row-contiguously: every store
        // instruction then writes whole rows of the wave's block, 16 bytes
        // per lane.  The ring is free once every wave has drained its loads
        // and crossed the barrier below.
        //   2-byte outputs: a lane's converted values are 8 bytes per block
        // and step; a lane swap (v_permlane16/32_swap) pairs two lanes'
        // pieces so that each lane holds 16 consecutive bytes of one row,
        // written with one 16-byte LDS write at strip_off (8-byte writes
        // measured bank conflicts in every layout).
        block_sync();
        if (WK > 1 && s.wk != 0) return;   // group 0 holds the sums; no barrier follows
        const int t = lane & 31, h = lane >> 5;
        const int mw = m0 + s.wm * WTM, nw = n0 + s.wn * WTN;
        uint8_t PG_LDS* strip = smem + s.wave * STRIP_BYTES;
        const bool full = (mw + WTM <= args.M) && (nw + WTN <= args.N);
#pragma unroll
        for (int fm = 0; fm < (B16 ? FM / 2 : FM); ++fm) {   // 32-row strips
            if constexpr (B16) {
                // 16x16 blocks 2 fm and 2 fm + 1: lane l holds row (l % 16),
                // columns 4 (l / 16) .. +3 of each.
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int row = 16 * half + (lane & 15), g = lane >> 4;
                    if constexpr (OSZ == 4) {
#pragma unroll
                        for (int fn = 0; fn < FN; ++fn)
                            *(i32x4 PG_LDS*)(strip + row * STRIP_ROW + (fn * 16 + 4 * g) * 4) = acc[2 * fm + half][fn];
                    } else {
                        // Blocks 2p and 2p + 1: after the swap (odd 16-lane
                        // groups' first block with even groups' second),
                        // group g holds columns 8 (g / 2) .. +7 of block
                        // 2p + (g % 2), i.e. 16-byte chunk 4p + 2 (g % 2) + g / 2.
#pragma unroll
                        for (int pb = 0; pb < FN / 2; ++pb) {
                            const f32x4 x = __builtin_bit_cast(f32x4, acc[2 * fm + half][2 * pb]);   // whole vector, then index
                            const f32x4 y = __builtin_bit_cast(f32x4, acc[2 * fm + half][2 * pb + 1]);
                            const i32x4 v = swap_pair<16>(cvt4_16(x[0], x[1], x[2], x[3]), cvt4_16(y[0], y[1], y[2], y[3]));
                            *(i32x4 PG_LDS*)(strip + strip_off(CPRS, row, epi16_chunk(pb, g))) = v;
                        }
                    }
                }
            } else
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                if constexpr (OSZ == 4) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *(i32x4 PG_LDS*)(strip + t * STRIP_ROW + (fn * 32 + 8 * q + 4 * h) * 4) = out4_32(acc[fm][fn], q);
                } else {
                    // q = 2j and 2j + 1: after the swap (upper half-wave's
                    // first with lower half-wave's second) half-wave h holds
                    // columns 8 (2j + h) .. +7, i.e. 16-byte chunk 4 fn + 2j + h.
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const i32x4 v = swap_pair<32>(out4_16(acc[fm][fn], 2 * j), out4_16(acc[fm][fn], 2 * j + 1));
                        *(i32x4 PG_LDS*)(strip + strip_off(CPRS, t, epi32_chunk(fn, j, h))) = v;
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 32 / ROWS_PER_STORE; ++i) {
                const int r = i * ROWS_PER_STORE + lane / LANES_PER_ROW;
                const int cc = lane % LANES_PER_ROW;                       // 16-byte chunk of the row
                const int c = cc * (kChunk / OSZ);                          // column in the wave block
                const i32x4 v = *(const i32x4 PG_LDS*)(strip + (OSZ == 2 ? strip_off(CPRS, r, cc) : r * STRIP_ROW + cc * kChunk));
                const int m = mw + fm * 32 + r, n = nw + c;
                uint8_t* dst = (uint8_t*)args.C + ((int64_t)m * args.ldc + n) * OSZ;
                if (full) {
                    // C is written once and not read here: stream it past the caches.
                    __builtin_nontemporal_store(v, (i32x4*)dst);
                } else if (m < args.M) {
                    store_part(dst, n, args.N, v);
                }
            }
        }
    }

    // Two lanes' 8-byte pieces into one lane's 16 bytes: x and y are the
    // lane's pieces of two blocks (steps); v_permlane<W>_swap exchanges the
    // odd W-lane groups' x with the even groups' y, so even groups return
    // (x, x of the next group) and odd groups (y of the previous group, y).
    template <int W>
    __device__ static __forceinline__ i32x4 swap_pair(i32x2 x, i32x2 y) {
        uint32_t a0 = (uint32_t)x[0], a1 = (uint32_t)x[1], b0 = (uint32_t)y[0], b1 = (uint32_t)y[1];
        if constexpr (W == 16) {
            const auto r0 = __builtin_amdgcn_permlane16_swap(a0, b0, false, false);
            const auto r1 = __builtin_amdgcn_permlane16_swap(a1, b1, false, false);
            a0 = r0[0]; b0 = r0[1]; a1 = r1[0]; b1 = r1[1];
        } else {
            const auto r0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
            const auto r1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
            a0 = r0[0]; b0 = r0[1]; a1 = r1[0]; b1 = r1[1];
        }
        return i32x4{(int)a0, (int)a1, (int)b0, (int)b1};
    }

    // Staging strip of the epilogue: 32 rows of one wave's block; 4-byte
    // outputs in rows padded so that the rows written at one column fall in
    // different LDS banks (see strip_row_bytes), 2-byte outputs placed by
    // strip_off.
    static constexpr int STRIP_ROW = strip_row_bytes(DT, TC);
    static constexpr int STRIP_BYTES = 32 * STRIP_ROW;
    static constexpr int CPRS = WTN * OSZ / kChunk;     // 16-byte chunks per strip row
    static_assert(OSZ == 4 || CPRS == 16 || CPRS == 8 || CPRS == 4, "2-byte strip layout");
    static constexpr int LANES_PER_ROW = WTN * OSZ / kChunk;
    static constexpr int ROWS_PER_STORE = 64 / LANES_PER_ROW;
    static_assert(64 % LANES_PER_ROW == 0 && 32 % ROWS_PER_STORE == 0, "epilogue store shape");
    static_assert(STRIP_BYTES * WM * WN <= LDS && (SPLIT ? 3 * A_BYTES + 2 * B_BYTES : SLOT * SLOTS) <= LDS,
                  "LDS layout");

    // Store the chunk v (16 bytes, columns n ..) of a row on the right edge:
    // whole if it lies inside C, else element by element.
    __device__ static __forceinline__ void store_part(uint8_t* dst, int n, int N, const i32x4 v) {
        constexpr int E = kChunk / OSZ;
        if (n + E <= N) {
            *(i32x4*)dst = v;
        } else if constexpr (OSZ == 4) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n + e < N) *(int*)(dst + e * 4) = v[e];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < N) *(uint16_t*)(dst + e * 2) = (uint16_t)((uint32_t)v[e >> 1] >> (16 * (e & 1)));
        }
    }

    // Four consecutive outputs of one row as stored: int32/fp32 as they are,
    // fp16/bf16 rounded to nearest even by the hardware conversion.
    __device__ static __forceinline__ i32x4 out4_32(const acc_t& a, int q) {
        const i32x16 ai = __builtin_bit_cast(i32x16, a);   // whole-vector cast
        return i32x4{ai[4 * q], ai[4 * q + 1], ai[4 * q + 2], ai[4 * q + 3]};
    }
    __device__ static __forceinline__ i32x2 out4_16(const acc_t& a, int q) {
        return cvt4_16(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
    }
    // a + b as accumulator words (int32 for int8, fp32 otherwise).
    __device__ static __forceinline__ i32x4 add_acc(const i32x4 a, const i32x4 b) {
        if constexpr (DT == DT_I8) {
            return a + b;
        } else {
            typedef float f32x4 __attribute__((ext_vector_type(4)));
            return __builtin_bit_cast(i32x4, __builtin_bit_cast(f32x4, a) + __builtin_bit_cast(f32x4, b));
        }
    }
    // C[m][n .. n+3] from four accumulator words: converted to the output
    // type, masked at column N.
    __device__ static __forceinline__ void store_out4(const GemmArgs& args, int m, int n, const i32x4 w) {
        uint8_t* dst = (uint8_t*)args.C + ((int64_t)m * args.ldc + n) * OSZ;
        if constexpr (OSZ == 4) {
            if (n + 4 <= args.N) {
                __builtin_nontemporal_store(w, (i32x4*)dst);
            } else {
                for (int e = 0; e < 4; ++e)
                    if (n + e < args.N) *(int*)(dst + 4 * e) = w[e];
            }
        } else {
            typedef float f32x4 __attribute__((ext_vector_type(4)));
            const f32x4 f = __builtin_bit_cast(f32x4, w);
            const i32x2 v = cvt4_16(f[0], f[1], f[2], f[3]);
            if (n + 4 <= args.N) {
                __builtin_nontemporal_store(v, (i32x2*)dst);
            } else {
                for (int e = 0; e < 4; ++e)
                    if (n + e < args.N) *(uint16_t*)(dst + 2 * e) = (uint16_t)((uint32_t)v[e >> 1] >> (16 * (e & 1)));
            }
        }
    }
    // Four fp32 values rounded to the 16-bit output type (nearest even), packed.
    __device__ static __forceinline__ i32x2 cvt4_16(float a0, float a1, float a2, float a3) {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        const f32x2 lo = {a0, a1}, hi = {a2, a3};
        if constexpr (DT == DT_BF16) {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            return i32x2{__builtin_bit_cast(int, __builtin_convertvector(lo, bf16x2)),
                         __builtin_bit_cast(int, __builtin_convertvector(hi, bf16x2))};
        } else {
            typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
            return i32x2{__builtin_bit_cast(int, __builtin_convertvector(lo, f16x2)),
                         __builtin_bit_cast(int, __builtin_convertvector(hi, f16x2))};
        }
    }

};

template <int DT, int LAYOUT, int TC, int STAGES, int VARIANT>
__global__ void __launch_bounds__(threads(TC), 1)
pipegemm_kernel(GemmArgs args) {
    typedef Gemm<DT, LAYOUT, TC, STAGES, VARIANT> G;
    __shared__ __attribute__((aligned(16))) uint8_t smem_raw[G::LDS];
    // Field-by-field copy: keeps every argument a uniform (scalar) value.
    GemmArgs a;
    a.A = args.A; a.B = args.B; a.C = args.C;
    a.lda = args.lda; a.ldb = args.ldb; a.ldc = args.ldc;
    a.M = args.M; a.N = args.N; a.K = args.K;
    a.tiles_m = args.tiles_m; a.tiles_n = args.tiles_n; a.splits = args.splits; a.sk_tiles = args.sk_tiles;
    a.ws = args.ws;
    G::run(a, (uint8_t PG_LDS*)smem_raw);
}

}  // namespace pg

#endif
