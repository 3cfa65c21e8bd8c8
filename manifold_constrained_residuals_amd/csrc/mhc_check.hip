// mhc_check.hip -- the environment switches, read on every call.
//
// MHC_CHECK_FINITE (anything but "" or "0"): every entry point that takes floating-point
// tensors scans its inputs before it launches anything (a non-finite input returns
// MHC_ERR_NONFINITE and computes nothing) and its outputs after its kernels (an overflow
// to Inf or a NaN returns MHC_ERR_NONFINITE with the outputs written).  A debugging aid,
// not part of the hot path: each scan synchronises the caller's stream, so the check is
// not for code under graph capture.
//
// MHC_FORCE_PATH ("vector" or "twopass"): the paths of the A/B comparisons (see
// force_path below).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "mhc_internal.hpp"

namespace mhc {
namespace {

// one flag per device: set to 1 by a scan that meets a NaN or an Inf
__device__ __align__(16) unsigned int nonfinite_flag[4];

__global__ __launch_bounds__(64) void k_flag_clear(unsigned int* flag)
{
    if (threadIdx.x == 0) flag[0] = 0u;
}

// rows x cols elements with row pitch ld (elements), fp32 or bf16; a lane that meets a
// non-finite element stores 1 into the flag (a plain vector store: every writer writes
// the same value)
__global__ __launch_bounds__(256) void k_scan_finite(const void* __restrict__ p, int64_t rows,
                                                     int64_t cols, int64_t ld, int bf16,
                                                     unsigned int* flag)
{
    const int64_t n = rows * cols;
    bool bad = false;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / cols, c = i - r * cols;
        const int64_t e = r * ld + c;
        uint32_t exp_bits;
        if (bf16) exp_bits = (uint32_t)(static_cast<const uint16_t*>(p)[e] >> 7) & 0xffu;
        else exp_bits = (__float_as_uint(static_cast<const float*>(p)[e]) >> 23) & 0xffu;
        bad |= exp_bits == 0xffu;                 // all exponent bits set: Inf or NaN
    }
    if (bad) flag[0] = 1u;
}

std::atomic<unsigned int*> flag_dev[64];
std::mutex flag_mu;

unsigned int* flag_ptr()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    unsigned int* p = flag_dev[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lk(flag_mu);
    p = flag_dev[dev].load(std::memory_order_relaxed);
    if (!p) {
        void* q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(nonfinite_flag)) != hipSuccess || !q) return nullptr;
        p = static_cast<unsigned int*>(q);
        flag_dev[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

// "vector": the vector kernels of the projections instead of the MFMA ones (which also
// rules out the single-read forward); "twopass": the forward read side in two passes
// over X instead of one; anything else: the default choice
int force_path()
{
    const char* e = std::getenv("MHC_FORCE_PATH");
    if (e && std::strcmp(e, "vector") == 0) return kPathVector;
    if (e && std::strcmp(e, "twopass") == 0) return kPathTwoPass;
    return kPathAuto;
}

bool check_finite_on()
{
    const char* e = std::getenv("MHC_CHECK_FINITE");
    return e && *e && std::strcmp(e, "0") != 0;
}

int scan_finite(hipStream_t s, std::initializer_list<FiniteSpan> spans)
{
    unsigned int* flag = flag_ptr();
    if (!flag) return -1;
    hipLaunchKernelGGL(k_flag_clear, dim3(1), dim3(64), 0, s, flag);
    for (const FiniteSpan& f : spans) {
        if (!f.p || f.rows <= 0 || f.cols <= 0) continue;
        const int64_t n = f.rows * f.cols;
        const int64_t blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
        hipLaunchKernelGGL(k_scan_finite, dim3((unsigned)blocks), dim3(256), 0, s, f.p, f.rows,
                           f.cols, f.ld, f.bf16 ? 1 : 0, flag);
    }
    unsigned int h = 0;
    if (hipGetLastError() != hipSuccess ||
        hipMemcpyAsync(&h, flag, sizeof(h), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return -1;
    return h ? 1 : 0;
}

}  // namespace mhc
