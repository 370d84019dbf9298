// ceiling_probe.hip -- attainable ceilings of one MI355X, to set beside the
// datasheet peaks: the matrix-core rate per input type when the MFMAs are
// fed from LDS the way the GEMM feeds them, and the HBM rate of a plain
// streaming read and copy.  Standalone program (no GEMM code): prints one
// "key: value" line per figure.
//
// MFMA ceiling.  One workgroup of 4 waves per CU; each wave keeps the GEMM's
// 4 x 4 blocks of 32 x 32 accumulators and, per k-step, reads 8 operand
// fragments (16 bytes per lane) from an LDS buffer of random values and
// issues the 16 MFMAs of the step -- the GEMM's ratio of LDS reads to MFMAs,
// without global memory traffic.  As in the GEMM, a step's fragments are read
// during the previous step's MFMAs, so LDS latency stays hidden.  A second
// figure per type (suffix _regs) feeds the MFMAs from two register-resident
// fragment sets used in turn, without LDS reads.  The data are random
// because the MFMA's power draw, and with it the clock the chip holds,
// depends on the operand bits; the effective clock is reported from
// s_memtime against the fixed 100 MHz s_memrealtime, and with it the share of
// cycles the matrix cores are busy (rate / (per-clock datasheet rate x clock)).
// A third figure (prefix mfma16_) runs the LDS-fed loop with 16x16 MFMA
// blocks, the GEMM's 256x256 2-3 stage direct instances' block shape, with
// the MFMA written as the GEMM writes it (tied inline assembly).
//
// HBM ceiling.  A 1 GiB buffer (four times the Infinity Cache) read once with
// 16-byte loads, each workgroup sweeping one contiguous block; the same
// buffer copied to a second one; and 1 GiB written with the 16-byte
// non-temporal stores the GEMM writes C with.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
#define LDSP __attribute__((address_space(3)))

enum { I8 = 0, F16 = 1, BF16 = 2, F32 = 3 };

template <int DT> struct Acc { typedef f32x16 type; };
template <> struct Acc<I8> { typedef i32x16 type; };

// acc += x * y over one 16-byte chunk per lane of each operand (fp32: four
// k = 2 instructions, as in the GEMM).
template <int DT>
__device__ __forceinline__ typename Acc<DT>::type mma(i32x4 x, i32x4 y, typename Acc<DT>::type c) {
    if constexpr (DT == BF16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, y), c, 0, 0, 0);
    } else if constexpr (DT == F16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, x), __builtin_bit_cast(f16x8, y), c, 0, 0, 0);
    } else if constexpr (DT == I8) {
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(x, y, c, 0, 0, 0);
    } else {
        const f32x4 xf = __builtin_bit_cast(f32x4, x), yf = __builtin_bit_cast(f32x4, y);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(xf[0], yf[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(xf[1], yf[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(xf[2], yf[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(xf[3], yf[3], c, 0, 0, 0);
        return c;
    }
}

// k covered by one 16-byte chunk per lane and 32 x 32 block
template <int DT> constexpr int chunk_k() { return DT == I8 ? 32 : DT == F32 ? 8 : 16; }

constexpr int kLdsUnits = 4096;   // 64 KiB of 16-byte units

// Random 16-byte unit i of workgroup b, with finite values of the type.
__device__ __forceinline__ i32x4 random_unit(int dt, uint32_t i, uint32_t b) {
    uint32_t x = i * 2654435761u + b * 40503u + 1u;
    i32x4 v;
    for (int e = 0; e < 4; ++e) {
        x ^= x << 13; x ^= x >> 17; x ^= x << 5;
        uint32_t w = x;
        if (dt == F16 || dt == BF16) w = (w & 0x83ff83ffu) | 0x38003800u;    // |v| in [0.5, 2)
        if (dt == BF16) w = (x & 0x807f807fu) | 0x3f003f00u;
        if (dt == F32) w = (w & 0x807fffffu) | 0x3f000000u;
        v[e] = (int)w;
    }
    return v;
}

// One k-step of a wave: the 16 MFMAs on fragments (x, y); with FEED, the
// next step's 8 fragments are read from LDS into (nx, ny), one after each of
// the first 8 MFMAs, while the matrix core works -- the GEMM's two-deep
// register pipeline, so no MFMA waits on a read issued in the same step.
template <int DT, bool FEED>
__device__ __forceinline__ void probe_step(typename Acc<DT>::type (&acc)[4][4], const i32x4 (&x)[4],
                                           const i32x4 (&y)[4], i32x4 (&nx)[4], i32x4 (&ny)[4],
                                           const i32x4 LDSP* lds, int next, int lane) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        acc[u / 4][u % 4] = mma<DT>(x[u % 4], y[u / 4], acc[u / 4][u % 4]);
        if (FEED && u < 8) {
            // unit index < 64 * 64 = kLdsUnits
            const int r = u & 3;
            if (u < 4) nx[r] = lds[((next * 8 + r) & 63) * 64 + lane];
            else ny[r] = lds[((next * 8 + 4 + r) & 63) * 64 + lane];
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// FEED: every k-step's operands come from LDS (random values), read one step
// ahead.  Without FEED the operands are two random fragment sets read once
// and used in turn: the matrix core alone, with operand bits that still
// change every step.
template <int DT, bool FEED>
__global__ void __launch_bounds__(256) mfma_ceiling(int iters, int* out, unsigned long long* clk) {
    typedef typename Acc<DT>::type acc_t;
    __shared__ __attribute__((aligned(16))) uint8_t lds_raw[kLdsUnits * 16];
    i32x4 LDSP* lds = (i32x4 LDSP*)lds_raw;
    const int tid = threadIdx.x, lane = tid & 63;
    for (int i = tid; i < kLdsUnits; i += 256) lds[i] = random_unit(DT, (uint32_t)i, blockIdx.x);
    __syncthreads();
    acc_t acc[4][4];
    for (int a = 0; a < 4; ++a)
        for (int b = 0; b < 4; ++b)
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0;
    i32x4 x0[4], y0[4], x1[4], y1[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        x0[a] = lds[a * 64 + lane];
        y0[a] = lds[(4 + a) * 64 + lane];
        x1[a] = lds[(8 + a) * 64 + lane];
        y1[a] = lds[(12 + a) * 64 + lane];
    }
    const unsigned long long t0 = __builtin_readcyclecounter(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; it += 2) {   // iters is even
        probe_step<DT, FEED>(acc, x0, y0, x1, y1, lds, it + 1, lane);
        probe_step<DT, FEED>(acc, x1, y1, x0, y0, lds, it + 2, lane);
    }
    const unsigned long long t1 = __builtin_readcyclecounter(), r1 = __builtin_amdgcn_s_memrealtime();
    int s = 0;
    for (int a = 0; a < 4; ++a)
        for (int b = 0; b < 4; ++b) {
            const i32x16 ai = __builtin_bit_cast(i32x16, acc[a][b]);   // whole-vector cast, then index
            s ^= ai[0] ^ ai[15];
        }
    out[blockIdx.x * 256 + tid] = s;
    if (tid == 0) {
        clk[blockIdx.x * 2] = t1 - t0;
        clk[blockIdx.x * 2 + 1] = r1 - r0;
    }
}

// The same loop with 16x16 MFMA blocks (16x16x32 for fp16/bf16, 16x16x64 for
// int8): 8 x 8 blocks per wave cover the same 128 x 128 accumulator tile, and
// each k-step reads 16 fragments for 64 MFMAs -- the same LDS bytes per
// multiply-add as the 32x32 loop.  Operands from LDS, read one step ahead.
//   The MFMA is written as the GEMM writes it: inline assembly with the
// accumulator tied in place in AGPRs.  (With the compiler's builtins the
// int8 loop moved its accumulators between registers at every step -- over
// 500 accvgpr moves per iteration -- and measured the copies, 75% busy.)
// The compiler sees no MFMA in these, so the kernel pads the hazards itself:
// a few wait states after the accumulators are set and before the first
// MFMA, and more than any MFMA result needs before they are read.
template <int DT>
__device__ __forceinline__ i32x4 mma16(i32x4 x, i32x4 y, i32x4 c) {
    if constexpr (DT == I8) {
        asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(c) : "v"(x), "v"(y));
    } else if constexpr (DT == BF16) {
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(x), "v"(y));
    } else {
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(x), "v"(y));
    }
    return c;
}

template <int DT>
__device__ __forceinline__ void probe_step16(i32x4 (&acc)[8][8], const i32x4 (&x)[8], const i32x4 (&y)[8],
                                             i32x4 (&nx)[8], i32x4 (&ny)[8], const i32x4 LDSP* lds, int next,
                                             int lane) {
#pragma unroll
    for (int u = 0; u < 64; ++u) {
        acc[u / 8][u % 8] = mma16<DT>(x[u % 8], y[u / 8], acc[u / 8][u % 8]);
        if (u % 4 == 0) {
            // unit index < 64 * 64 = kLdsUnits
            const int r = u / 4;
            if (r < 8) nx[r] = lds[((next * 16 + r) & 63) * 64 + lane];
            else ny[r - 8] = lds[((next * 16 + r) & 63) * 64 + lane];
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int DT>
__global__ void __launch_bounds__(256) mfma16_ceiling(int iters, int* out, unsigned long long* clk) {
    __shared__ __attribute__((aligned(16))) uint8_t lds_raw[kLdsUnits * 16];
    i32x4 LDSP* lds = (i32x4 LDSP*)lds_raw;
    const int tid = threadIdx.x, lane = tid & 63;
    for (int i = tid; i < kLdsUnits; i += 256) lds[i] = random_unit(DT, (uint32_t)i, blockIdx.x);
    __syncthreads();
    i32x4 acc[8][8];
    for (int a = 0; a < 8; ++a)
        for (int b = 0; b < 8; ++b) acc[a][b] = i32x4{0, 0, 0, 0};
    i32x4 x0[8], y0[8], x1[8], y1[8];
#pragma unroll
    for (int a = 0; a < 8; ++a) {
        x0[a] = lds[a * 64 + lane];
        y0[a] = lds[(8 + a) * 64 + lane];
        x1[a] = lds[(16 + a) * 64 + lane];
        y1[a] = lds[(24 + a) * 64 + lane];
    }
    const unsigned long long t0 = __builtin_readcyclecounter(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; it += 2) {   // iters is even
        asm volatile("s_nop 4" ::: "memory");   // accumulators set by ordinary moves before the loop
        probe_step16<DT>(acc, x0, y0, x1, y1, lds, it + 1, lane);
        probe_step16<DT>(acc, x1, y1, x0, y0, lds, it + 2, lane);
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");   // last MFMA results before they are read
    const unsigned long long t1 = __builtin_readcyclecounter(), r1 = __builtin_amdgcn_s_memrealtime();
    int s = 0;
    for (int a = 0; a < 8; ++a)
        for (int b = 0; b < 8; ++b) s ^= acc[a][b][0] ^ acc[a][b][3];
    out[blockIdx.x * 256 + tid] = s;
    if (tid == 0) {
        clk[blockIdx.x * 2] = t1 - t0;
        clk[blockIdx.x * 2 + 1] = r1 - r0;
    }
}

// Each workgroup reads (and for the copy, writes) one contiguous block of
// `per_wg` bytes, 4 x 16 bytes per lane per pass.
__global__ void __launch_bounds__(256) hbm_read(const i32x4* __restrict__ src, uint64_t per_wg, int* out) {
    const i32x4* p = src + (uint64_t)blockIdx.x * (per_wg / 16);
    i32x4 acc = {0, 0, 0, 0};
    for (uint64_t u = threadIdx.x; u < per_wg / 16; u += 4 * 256) {
        i32x4 v0 = p[u], v1 = p[u + 256], v2 = p[u + 512], v3 = p[u + 768];
        acc ^= v0 ^ v1 ^ v2 ^ v3;
    }
    if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x5a5a5a5a) out[threadIdx.x] = acc[0];
}

__global__ void __launch_bounds__(256) hbm_copy(const i32x4* __restrict__ src, i32x4* __restrict__ dst, uint64_t per_wg) {
    const uint64_t base = (uint64_t)blockIdx.x * (per_wg / 16);
    for (uint64_t u = threadIdx.x; u < per_wg / 16; u += 4 * 256) {
        i32x4 v0 = src[base + u], v1 = src[base + u + 256], v2 = src[base + u + 512], v3 = src[base + u + 768];
        dst[base + u] = v0;
        dst[base + u + 256] = v1;
        dst[base + u + 512] = v2;
        dst[base + u + 768] = v3;
    }
}

// Each workgroup writes one contiguous block with 16-byte non-temporal
// stores, the store the GEMM's epilogue uses for C.
__global__ void __launch_bounds__(256) hbm_write(i32x4* __restrict__ dst, uint64_t per_wg) {
    const uint64_t base = (uint64_t)blockIdx.x * (per_wg / 16);
    const i32x4 v = {(int)blockIdx.x, (int)threadIdx.x, 1, 2};
    for (uint64_t u = threadIdx.x; u < per_wg / 16; u += 4 * 256) {
        __builtin_nontemporal_store(v, dst + base + u);
        __builtin_nontemporal_store(v, dst + base + u + 256);
        __builtin_nontemporal_store(v, dst + base + u + 512);
        __builtin_nontemporal_store(v, dst + base + u + 768);
    }
}

#define CHECK(x)                                                                 \
    do {                                                                         \
        hipError_t e_ = (x);                                                     \
        if (e_ != hipSuccess) {                                                  \
            std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));         \
            return 1;                                                            \
        }                                                                        \
    } while (0)

template <int DT, bool FEED>
int run_mfma(const char* name, double peak, int cus) {
    int* out;
    unsigned long long* clk;
    CHECK(hipMalloc(&out, (size_t)cus * 256 * sizeof(int)));
    CHECK(hipMalloc(&clk, (size_t)cus * 2 * sizeof(unsigned long long)));
    const int iters = DT == F32 ? 2000 : 8000;
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    for (int w = 0; w < 3; ++w) mfma_ceiling<DT, FEED><<<dim3(cus), dim3(256)>>>(iters, out, clk);
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    const int reps = 5;
    for (int r = 0; r < reps; ++r) mfma_ceiling<DT, FEED><<<dim3(cus), dim3(256)>>>(iters, out, clk);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    ms /= reps;
    std::vector<unsigned long long> h((size_t)cus * 2);
    CHECK(hipMemcpy(h.data(), clk, h.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost));
    double cyc = 0, rt = 0;
    for (int b = 0; b < cus; ++b) {
        cyc += (double)h[2 * b];
        rt += (double)h[2 * b + 1];
    }
    const double ghz = cyc / (rt / 100e6) / 1e9;
    // per wave and iteration: 16 blocks of 32 x 32 x chunk_k multiply-adds
    const double ops = 2.0 * 16 * 32 * 32 * chunk_k<DT>() * 4 * (double)cus * iters;
    const double t = ops / (ms * 1e-3) / 1e12;
    // matrix-core busy share: the rate against the datasheet's per-clock rate at the measured clock
    const double busy = t / (peak * ghz / 2.4);
    std::printf("mfma_%s%s: %.1f %s, effective clock %.3f GHz, %.1f%% of the %.1f datasheet peak, "
                "matrix cores busy %.1f%% of cycles\n", name, FEED ? "" : "_regs", t,
                DT == I8 ? "TOP/s" : "TFLOP/s", ghz, 100.0 * t / peak, peak, 100.0 * busy);
    CHECK(hipFree(out));
    CHECK(hipFree(clk));
    return 0;
}

template <int DT>
int run_mfma16(const char* name, double peak, int cus) {
    int* out;
    unsigned long long* clk;
    CHECK(hipMalloc(&out, (size_t)cus * 256 * sizeof(int)));
    CHECK(hipMalloc(&clk, (size_t)cus * 2 * sizeof(unsigned long long)));
    const int iters = 4000;   // one iteration: k = 32 (int8: 64) over the 128 x 128 tile
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    for (int w = 0; w < 3; ++w) mfma16_ceiling<DT><<<dim3(cus), dim3(256)>>>(iters, out, clk);
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    const int reps = 5;
    for (int r = 0; r < reps; ++r) mfma16_ceiling<DT><<<dim3(cus), dim3(256)>>>(iters, out, clk);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    ms /= reps;
    std::vector<unsigned long long> h((size_t)cus * 2);
    CHECK(hipMemcpy(h.data(), clk, h.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost));
    double cyc = 0, rt = 0;
    for (int b = 0; b < cus; ++b) {
        cyc += (double)h[2 * b];
        rt += (double)h[2 * b + 1];
    }
    const double ghz = cyc / (rt / 100e6) / 1e9;
    const double ops = 2.0 * 64 * 16 * 16 * (DT == I8 ? 64 : 32) * 4 * (double)cus * iters;
    const double t = ops / (ms * 1e-3) / 1e12;
    const double busy = t / (peak * ghz / 2.4);
    std::printf("mfma16_%s: %.1f %s, effective clock %.3f GHz, %.1f%% of the %.1f datasheet peak, "
                "matrix cores busy %.1f%% of cycles\n", name, t, DT == I8 ? "TOP/s" : "TFLOP/s", ghz,
                100.0 * t / peak, peak, 100.0 * busy);
    CHECK(hipFree(out));
    CHECK(hipFree(clk));
    return 0;
}

}  // namespace

int main() {
    int dev = 0, cus = 0;
    CHECK(hipGetDevice(&dev));
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    std::printf("compute_units: %d\n", cus);
    if (run_mfma<I8, true>("int8", 5033.2, cus) || run_mfma<F16, true>("fp16", 2516.6, cus) ||
        run_mfma<BF16, true>("bf16", 2516.6, cus) || run_mfma<F32, true>("fp32", 157.3, cus))
        return 1;
    if (run_mfma16<I8>("int8", 5033.2, cus) || run_mfma16<F16>("fp16", 2516.6, cus) ||
        run_mfma16<BF16>("bf16", 2516.6, cus))
        return 1;
    if (run_mfma<I8, false>("int8", 5033.2, cus) || run_mfma<F16, false>("fp16", 2516.6, cus) ||
        run_mfma<BF16, false>("bf16", 2516.6, cus))
        return 1;

    const uint64_t bytes = (uint64_t)1 << 30;
    const int wgs = 4096;                       // 256 KiB per workgroup
    const uint64_t per_wg = bytes / wgs;        // a multiple of 4 * 256 * 16 bytes
    i32x4 *src, *dst;
    int* out;
    CHECK(hipMalloc(&src, bytes));
    CHECK(hipMalloc(&dst, bytes));
    CHECK(hipMalloc(&out, 256 * sizeof(int)));
    CHECK(hipMemset(src, 1, bytes));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    float ms;
    for (int w = 0; w < 3; ++w) hipLaunchKernelGGL(hbm_read, dim3(wgs), dim3(256), 0, 0, src, per_wg, out);
    CHECK(hipEventRecord(e0));
    for (int r = 0; r < 10; ++r) hipLaunchKernelGGL(hbm_read, dim3(wgs), dim3(256), 0, 0, src, per_wg, out);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    std::printf("hbm_read: %.1f GB/s (1 GiB, 16-byte loads)\n", (double)bytes * 10 / (ms * 1e-3) / 1e9);
    for (int w = 0; w < 3; ++w) hipLaunchKernelGGL(hbm_copy, dim3(wgs), dim3(256), 0, 0, src, dst, per_wg);
    CHECK(hipEventRecord(e0));
    for (int r = 0; r < 10; ++r) hipLaunchKernelGGL(hbm_copy, dim3(wgs), dim3(256), 0, 0, src, dst, per_wg);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    std::printf("hbm_copy: %.1f GB/s (read + write bytes, 1 GiB each way)\n", 2.0 * bytes * 10 / (ms * 1e-3) / 1e9);
    for (int w = 0; w < 3; ++w) hipLaunchKernelGGL(hbm_write, dim3(wgs), dim3(256), 0, 0, dst, per_wg);
    CHECK(hipEventRecord(e0));
    for (int r = 0; r < 10; ++r) hipLaunchKernelGGL(hbm_write, dim3(wgs), dim3(256), 0, 0, dst, per_wg);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    std::printf("hbm_write: %.1f GB/s (1 GiB, 16-byte non-temporal stores)\n", (double)bytes * 10 / (ms * 1e-3) / 1e9);
    CHECK(hipFree(src));
    CHECK(hipFree(dst));
    CHECK(hipFree(out));
    return 0;
}
