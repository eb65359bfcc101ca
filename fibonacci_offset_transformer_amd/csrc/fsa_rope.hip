// Rotation pass of libfsa (gfx950): rotary position embedding of bf16 rows into a
// workspace; with its launcher.
#include "fsa_device.h"

namespace fsa {
namespace {

// ----------------------------------------------------------------------------
// rotary position embedding
// ----------------------------------------------------------------------------

// Rotates bf16 rows into bf16 rows: one thread per 16-byte chunk (channel pairs
// 4c .. 4c + 3 of one row, eight threads per row), the same chunk of every tensor, so
// that each table entry is read once. Rows are addressed as (head, position) with
// blockIdx.y the head, so positions need no division.
__global__ void __launch_bounds__(kThreads) rope_kernel(const RopeParams p) {
    const int idx = blockIdx.x * kThreads + threadIdx.x;  // chunk within the head
    const int pos = idx >> 3, c = idx & 7;
    if (pos >= p.n) return;
    const int64_t row = ((int64_t)p.head0 + blockIdx.y) * p.n + pos;
    const f32x4_t *tab = reinterpret_cast<const f32x4_t *>(p.table + ((int64_t)pos * 32 + 4 * c) * 2);
    const f32x4_t t01 = tab[0], t23 = tab[1];  // (cos, sin) of pairs 4c, 4c + 1, then 4c + 2, 4c + 3
    u32x4_t xv[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
        if (t < p.count)
            xv[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p.x[t] + row * 64 + 8 * c));
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        if (t < p.count) {
            u32x4_t ov;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const f32x4_t &tt = k < 2 ? t01 : t23;
                const int j = 2 * (k & 1);
                float re, ro;
                rope_pair(tt[j], tt[j + 1], bf16_lo(xv[t][k]), bf16_hi(xv[t][k]), re, ro);
                ov[k] = pack_bf16(re, ro);
            }
            *reinterpret_cast<u32x4_t *>(p.out[t] + row * 64 + 8 * c) = ov;
        }
    }
}

}  // namespace

hipError_t launch_rope(const RopeParams &p, hipStream_t s) {
    const int64_t chunks = (int64_t)p.n * 8;  // per head
    const int64_t heads = p.rows / p.n;
    constexpr int64_t kMaxY = 65535;  // heads per launch (grid y)
    for (int64_t h0 = 0; h0 < heads; h0 += kMaxY) {
        const dim3 grid((unsigned)((chunks + kThreads - 1) / kThreads), (unsigned)std::min(kMaxY, heads - h0));
        RopeParams a = p;
        a.head0 = h0;
        void *args[] = {&a};
        const hipError_t e =
            hipLaunchKernel(reinterpret_cast<const void *>(&rope_kernel), grid, dim3(kThreads), args, 0, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace fsa
