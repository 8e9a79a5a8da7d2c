// Measurements of gfx950 behaviour that the tiled kernels' layout rests on, re-runnable through
// tests/test_gpu_probes.py (test infrastructure: nothing here is part of the library).
//
//  * LDS reads: 16 waves per CU, each wave's 4 slots of 16 lanes reading one 256-byte row apiece
//    with ds_read_b128 (lane j reads 16-byte chunk j at position j ^ (row & mask)), 8 reads in
//    flight per lane;
//  * LDS writes: ds_write_b128 of consecutive rows by consecutive lanes, one chunk position per
//    instruction, at position chunk ^ (row & mask) (the staging pattern);
//  * VALU issue rates of the instruction forms a tiled step uses: 8 independent chains per wave,
//    16 waves per CU.
// Every LDS address stays below 640 rows x 256 bytes (the 160 KB allocation); the loads wait for
// their results inside the same asm block.
#include <hip/hip_runtime.h>

namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 1024;
constexpr int kRows = 600;            // rows addressed (of 640 allocated)
constexpr size_t kLds = 640 * 256;    // bytes of dynamic LDS

__global__ __launch_bounds__(kThreads) void lds_read_kernel(int iters, unsigned mask) {
    extern __shared__ float lds[];
    for (int i = threadIdx.x; i < static_cast<int>(kLds / 4); i += kThreads) lds[i] = static_cast<float>(i);
    __syncthreads();
    const unsigned lane = threadIdx.x & 63, slot = lane >> 4, j = lane & 15, w = threadIdx.x >> 6;
    unsigned a[8];
    for (int m = 0; m < 8; ++m) {
        const unsigned r = (w * 131u + m * 977u + slot * 211u + 13u) % kRows;
        a[m] = r * 256 + 16 * (j ^ (r & mask));
    }
    for (int it = 0; it < iters; ++it) {
        f4 v0, v1, v2, v3, v4, v5, v6, v7;
        asm volatile(
            "ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\tds_read_b128 %3, %11\n\t"
            "ds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\tds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=v"(v0), "=v"(v1), "=v"(v2), "=v"(v3), "=v"(v4), "=v"(v5), "=v"(v6), "=v"(v7)
            : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]));
        asm volatile("" ::"v"(v0), "v"(v1), "v"(v2), "v"(v3), "v"(v4), "v"(v5), "v"(v6), "v"(v7));
    }
}

__global__ __launch_bounds__(kThreads) void lds_write_kernel(int iters, unsigned mask) {
    extern __shared__ float lds[];
    const unsigned lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    unsigned a[8];
    for (int m = 0; m < 8; ++m) {
        const unsigned row = (w * 64 + lane + m * 37u) % kRows, q = (m * 5u + w) & 15u;
        a[m] = row * 256 + 16 * (q ^ (row & mask));
    }
    f4 v = {1.f, 2.f, 3.f, static_cast<float>(threadIdx.x)};
    for (int it = 0; it < iters; ++it) {
        asm volatile(
            "ds_write_b128 %0, %8\n\tds_write_b128 %1, %8\n\tds_write_b128 %2, %8\n\tds_write_b128 %3, %8\n\t"
            "ds_write_b128 %4, %8\n\tds_write_b128 %5, %8\n\tds_write_b128 %6, %8\n\tds_write_b128 %7, %8\n\t"
            "s_waitcnt lgkmcnt(0)" ::"v"(a[0]),
            "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(v));
    }
}

// MODE 0 v_fmac_f32, 1 v_fmac_f32 with DPP row_newbcast, 2 v_mov_b32 with DPP row_newbcast,
// 3 v_xor_b32 with DPP row_newbcast
template <int MODE>
__global__ __launch_bounds__(kThreads) void valu_kernel(float *out, int iters, unsigned seed) {
    float a[8];
    unsigned u[8];
    for (int i = 0; i < 8; ++i) {
        a[i] = static_cast<float>(threadIdx.x + i);
        u[i] = seed * (threadIdx.x + 17 * i);
    }
    const unsigned v = seed ^ threadIdx.x;
    asm volatile("s_nop 4" ::"v"(v));  // wait states between the writes above and the first DPP read
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if constexpr (MODE == 0)
                asm volatile("v_fmac_f32 %0, %1, %2" : "+v"(a[i]) : "v"(a[(i + 1) & 7]), "v"(v));
            if constexpr (MODE == 1)
                asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:1 row_mask:0xf bank_mask:0xf bound_ctrl:1"
                             : "+v"(a[i]) : "v"(v), "v"(a[(i + 1) & 7]));
            if constexpr (MODE == 2)
                asm volatile("v_mov_b32_dpp %0, %1 row_newbcast:1 row_mask:0xf bank_mask:0xf bound_ctrl:1"
                             : "=v"(u[i]) : "v"(v));
            if constexpr (MODE == 3)
                asm volatile("v_xor_b32_dpp %0, %0, %1 row_newbcast:1 row_mask:0xf bank_mask:0xf bound_ctrl:1"
                             : "+v"(u[i]) : "v"(v));
        }
    }
    float s = 0;
    for (int i = 0; i < 8; ++i) s += a[i] + static_cast<float>(u[i]);
    if (s == 1.2345f) out[threadIdx.x] = s;  // keeps the chains live; never true for these inputs
}

template <typename Launch>
int time_ms(Launch launch, float &ms) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return 1;
    launch(10);
    if (hipDeviceSynchronize() != hipSuccess) return 1;
    (void)hipEventRecord(a);
    launch(0);
    (void)hipEventRecord(b);
    if (hipEventSynchronize(b) != hipSuccess) return 1;
    (void)hipEventElapsedTime(&ms, a, b);
    (void)hipEventDestroy(a);
    (void)hipEventDestroy(b);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

constexpr int kGrid = 256;
constexpr int kIters = 4000;

}  // namespace

// LDS bytes per clock per CU (at 2.4 GHz) of the read pattern with the given swizzle mask; 0 on
// success.
extern "C" int probe_lds_read(unsigned mask, double *bytes_per_clk_cu) {
    if (mask > 15 || !bytes_per_clk_cu) return 2;
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(&lds_read_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLds)) != hipSuccess)
        return 1;
    float ms = 0;
    const int s = time_ms([&](int warm) {
        hipLaunchKernelGGL(lds_read_kernel, dim3(kGrid), dim3(kThreads), kLds, 0, warm ? warm : kIters, mask);
    }, ms);
    *bytes_per_clk_cu = double(kGrid) * 16 * kIters * 8 * 1024.0 / (ms * 1e-3) / 256 / 2.4e9;
    return s;
}

// The same for the staging write pattern.
extern "C" int probe_lds_write(unsigned mask, double *bytes_per_clk_cu) {
    if (mask > 15 || !bytes_per_clk_cu) return 2;
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(&lds_write_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLds)) != hipSuccess)
        return 1;
    float ms = 0;
    const int s = time_ms([&](int warm) {
        hipLaunchKernelGGL(lds_write_kernel, dim3(kGrid), dim3(kThreads), kLds, 0, warm ? warm : kIters, mask);
    }, ms);
    *bytes_per_clk_cu = double(kGrid) * 16 * kIters * 8 * 1024.0 / (ms * 1e-3) / 256 / 2.4e9;
    return s;
}

// Wave-instructions per clock per CU (at 2.4 GHz) of instruction form `mode` (see valu_kernel).
extern "C" int probe_valu_rate(int mode, double *wave_instr_per_clk_cu) {
    if (mode < 0 || mode > 3 || !wave_instr_per_clk_cu) return 2;
    float *out = nullptr;
    if (hipMalloc(&out, kThreads * sizeof(float)) != hipSuccess) return 1;
    float ms = 0;
    int s = 0;
    auto run = [&](auto kernel) {
        return time_ms([&](int warm) {
            hipLaunchKernelGGL(kernel, dim3(kGrid), dim3(kThreads), 0, 0, out, warm ? warm : kIters, 2654435761u);
        }, ms);
    };
    switch (mode) {
        case 0: s = run(valu_kernel<0>); break;
        case 1: s = run(valu_kernel<1>); break;
        case 2: s = run(valu_kernel<2>); break;
        default: s = run(valu_kernel<3>); break;
    }
    (void)hipFree(out);
    *wave_instr_per_clk_cu = double(kGrid) * 16 * kIters * 8 / (ms * 1e-3) / 256 / 2.4e9;
    return s;
}
