// The backward for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation): fsa_backward with its
// two workspaces (D, and the pair weights, tokens and status word of the window path)
// taken from a static device array of this library instead of from the caller.
//
// The array is a file-scope __device__ variable: every GPU the library runs on holds its
// own copy, at its own address, until the process ends. Host code never uses the array's
// name as an address (on the host that name is only a stand-in); it looks the device
// address up once per device with hipGetSymbolAddress, with that device current, and
// passes that address to the kernels.
#include <mutex>

#include "fsa_internal.h"

namespace fsa {

const uint64_t kScratchBytes = 32ull << 20;  // 32 MiB per device

namespace {

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_address(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace fsa

extern "C" fsa_status_t fsa_backward_noalloc(fsa_dtype_t dt, fsa_dtype_t out_dt, const void *q, const void *k,
                                             const void *v, const void *o, const float *lse, const void *dout,
                                             void *dq, void *dk, void *dv, int32_t B, int32_t H, int32_t N, int32_t d,
                                             float scale, fsa_base_t base, double alpha, int32_t w, int32_t R,
                                             void *stream) {
    // sizes of the two workspaces (this also validates the shape and table arguments)
    uint64_t pair_bytes = 0;
    fsa_status_t st = fsa_backward_workspace_bytes(dt, B, H, N, d, base, alpha, w, R, &pair_bytes);
    if (st != FSA_OK) return st;
    if (static_cast<int64_t>(B) * H * N == 0)  // an empty problem: nothing to hold
        return fsa_backward(dt, out_dt, q, k, v, o, lse, dout, dq, dk, dv, nullptr, nullptr, 0, B, H, N, d, scale,
                            base, alpha, w, R, stream);
    const uint64_t delta_bytes = fsa::align256(4ull * static_cast<uint64_t>(B) * H * N);
    if (delta_bytes + pair_bytes > fsa::kScratchBytes) {
        char msg[256];
        snprintf(msg, sizeof msg,
                 "this problem needs %llu bytes of scratch (D and pair weights); the library's static scratch "
                 "holds %llu: use fsa_backward with caller workspaces",
                 static_cast<unsigned long long>(delta_bytes + pair_bytes),
                 static_cast<unsigned long long>(fsa::kScratchBytes));
        return fsa::set_error(FSA_E_CAPACITY, msg);
    }
    void *base_ptr = nullptr;
    const hipError_t e = fsa::scratch_address(&base_ptr);
    if (e != hipSuccess) {
        char msg[256];
        snprintf(msg, sizeof msg, "looking up the scratch array failed: %s", hipGetErrorString(e));
        return fsa::set_error(FSA_E_HIP, msg);
    }
    char *b = static_cast<char *>(base_ptr);
    return fsa_backward(dt, out_dt, q, k, v, o, lse, dout, dq, dk, dv, reinterpret_cast<float *>(b),
                        pair_bytes > 0 ? b + delta_bytes : nullptr, pair_bytes, B, H, N, d, scale, base, alpha, w, R,
                        stream);
}
