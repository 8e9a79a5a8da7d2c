// layout_kernels.h -- part of libsnack_coo's device code, included once by snack_coo.hip (after the
// headers before it in that file's include list, whose definitions it uses).
// Layout copies: batch-major activations to the feature-major operand that the
// untiled gathers read (K10), memory clears and the bias gradient.
#pragma once

namespace {

// ---------------------------------------------------------------- layout
// in [B][F] (batch-major, fp32 or bf16)  ->  out [F+1][Bp] fp32 (feature-major, Bp >= B; columns
// B..Bp-1 zero), row F zero (gathers of a missing entry point there instead of being masked).
// Up to two tensors per launch (blockIdx.z; the backward pass transposes X and dY together).
// A workgroup moves a tile of 32 features x 64 batch rows through LDS.
constexpr int kTf = 32, kTb = 64;

// Any F and B: each thread issues its eight scalar loads (128-byte row segments per 32 lanes)
// before its stores; the tile's output is one contiguous run per feature.
template <typename InT>
__global__ __launch_bounds__(kBlock) void to_feature_major_kernel(const InT *__restrict__ in0,
                                                                  float *__restrict__ out0, int64_t F0,
                                                                  const InT *__restrict__ in1,
                                                                  float *__restrict__ out1, int64_t F1,
                                                                  int64_t B, int64_t Bp) {
    __shared__ float tile[kTb][kTf + 1];
    const InT *__restrict__ in = blockIdx.z == 0 ? in0 : in1;
    float *__restrict__ out = blockIdx.z == 0 ? out0 : out1;
    const int64_t F = blockIdx.z == 0 ? F0 : F1;
    const int64_t f0 = static_cast<int64_t>(blockIdx.x) * kTf;
    if (f0 >= F && !(blockIdx.x == 0)) return;  // uniform per workgroup, before the barrier
    const int64_t b0 = static_cast<int64_t>(blockIdx.y) * kTb;
    const int tx = threadIdx.x % kTf, ty = threadIdx.x / kTf;  // 32 x 8
    const int nb = static_cast<int>(max<int64_t>(0, min<int64_t>(kTb, B - b0)));
    const int nbp = static_cast<int>(min<int64_t>(kTb, Bp - b0));  // with the zero columns
    const int nf = static_cast<int>(max<int64_t>(0, min<int64_t>(kTf, F - f0)));
    if (blockIdx.x == 0 && static_cast<int>(threadIdx.x) < nbp) out[F * Bp + b0 + threadIdx.x] = 0.f;
    constexpr int K = kTb / (kBlock / kTf);  // 8 rows per thread
    float v[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
        const int bb = ty + (kBlock / kTf) * i;
        v[i] = (bb < nb && tx < nf) ? load_act(in, (b0 + bb) * F + f0 + tx) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < K; ++i) tile[ty + (kBlock / kTf) * i][tx] = v[i];
    __syncthreads();
    for (int li = threadIdx.x; li < nf * nbp; li += kBlock) {  // rows nb..nbp-1 of the tile are zero
        const int ff = li / nbp, bb = li % nbp;
        out[(f0 + ff) * Bp + b0 + bb] = tile[bb][ff];
    }
}

__device__ __forceinline__ float4 load_act4(const float *p, int64_t i) {
    return *reinterpret_cast<const float4 *>(p + i);
}
__device__ __forceinline__ float4 load_act4(const bf16_t *p, int64_t i) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p + i);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u), __uint_as_float(u.y << 16),
                       __uint_as_float(u.y & 0xFFFF0000u));
}

// F and Bp multiples of 4 (16-byte aligned rows): each thread loads two 4-feature vectors of
// two batch rows (zeros past B) and stores two 4-row vectors of two features, with no divisions.  LDS rows
// are padded to 33 floats: the 4 scalar writes and reads of a vector fall in distinct banks.
template <typename InT>
__global__ __launch_bounds__(kBlock) void to_feature_major4_kernel(const InT *__restrict__ in0,
                                                                   float *__restrict__ out0, int64_t F0,
                                                                   const InT *__restrict__ in1,
                                                                   float *__restrict__ out1, int64_t F1,
                                                                   int64_t B, int64_t Bp) {
    __shared__ float tile[kTb][kTf + 1];
    const InT *__restrict__ in = blockIdx.z == 0 ? in0 : in1;
    float *__restrict__ out = blockIdx.z == 0 ? out0 : out1;
    const int64_t F = blockIdx.z == 0 ? F0 : F1;
    const int64_t f0 = static_cast<int64_t>(blockIdx.x) * kTf;
    if (f0 >= F && !(blockIdx.x == 0)) return;  // uniform per workgroup, before the barrier
    const int64_t b0 = static_cast<int64_t>(blockIdx.y) * kTb;
    const int tid = threadIdx.x;
    if (blockIdx.x == 0 && b0 + tid < Bp && tid < kTb) out[F * Bp + b0 + tid] = 0.f;
    // load: thread -> batch row r = tid / 8 (+32), features 4 * (tid % 8) .. +3
    const int lc = 4 * (tid % (kTf / 4)), lr = tid / (kTf / 4);
    float4 v[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t b = b0 + lr + 32 * i, f = f0 + lc;
        v[i] = (b < B && f < F) ? load_act4(in, b * F + f) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        float *t = &tile[lr + 32 * i][lc];
        t[0] = v[i].x;
        t[1] = v[i].y;
        t[2] = v[i].z;
        t[3] = v[i].w;
    }
    __syncthreads();
    // store: thread -> feature ff = tid / 16 (+16), batch rows 4 * (tid % 16) .. +3
    const int sq = 4 * (tid % (kTb / 4)), sf = tid / (kTb / 4);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int ff = sf + 16 * i;
        const int64_t f = f0 + ff, b = b0 + sq;
        if (f < F && b < Bp)
            *reinterpret_cast<float4 *>(out + f * Bp + b) =
                make_float4(tile[sq][ff], tile[sq + 1][ff], tile[sq + 2][ff], tile[sq + 3][ff]);
    }
}


__global__ __launch_bounds__(kBlock) void zero_kernel(float *__restrict__ p, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// ---------------------------------------------------------------- bias gradient
template <typename InT>
__global__ __launch_bounds__(kBlock) void bias_grad_kernel(int64_t O, int64_t B, const InT *__restrict__ dY,
                                                           float *__restrict__ db) {
    const int64_t o = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
    if (o >= O) return;
    float s = 0.f;
    for (int64_t b = 0; b < B; ++b) s += load_act(dY, b * O + o);
    db[o] = s;
}

}  // namespace
