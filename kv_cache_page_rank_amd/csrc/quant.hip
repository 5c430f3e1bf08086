// Stand-alone quantiser: fp32 summaries -> int8 / int4 codes and scales for
// every unit (block, KV head) of the pools (technical summary, section 2,
// Kwantisatie).  One 256-thread workgroup per unit stages the unit in LDS and
// runs the same quantize_unit as the summary builder's quantised output.
#include "device_common.hpp"
#include "launchers.hpp"
#include "quant.hpp"

namespace locks {

namespace {

constexpr int kQuantThreads = 256;

template <int P, int D>
__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(const QuantParams a) {
    __shared__ float mu[D];
    __shared__ float basis[16 * D];
    __shared__ float coef[P * 16];
    __shared__ float amax[1 + 2 * 16], qs[1 + 2 * 16];
    const int t = threadIdx.x;
    const int r = a.rank;
    const size_t u = blockIdx.x;
    for (int i = t; i < D; i += kQuantThreads) mu[i] = a.mu[u * D + i];
    for (int i = t; i < r * D; i += kQuantThreads) basis[i] = a.basis[u * r * D + i];
    for (int i = t; i < P * r; i += kQuantThreads) coef[i] = a.coef[u * P * r + i];
    __syncthreads();
    quantize_unit<P, D, kQuantThreads>(mu, basis, D, coef, r, r, a.mu_q + u * D,
                                       a.basis_q + u * r * (D / 2), a.coef_q + u * P * r,
                                       a.scales + u * (1 + 2 * r), amax, qs, t);
}

template <int P, int D>
hipError_t launch_pd(const QuantParams& p, hipStream_t s) {
    if (p.units <= 0) return hipSuccess;
    hipLaunchKernelGGL((quantize_kernel<P, D>), dim3((unsigned)p.units), dim3(kQuantThreads), 0,
                       s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantParams& p, hipStream_t s) {
    if (p.page_size == 16 && p.head_dim == 64) return launch_pd<16, 64>(p, s);
    if (p.page_size == 16 && p.head_dim == 128) return launch_pd<16, 128>(p, s);
    if (p.page_size == 64 && p.head_dim == 64) return launch_pd<64, 64>(p, s);
    return launch_pd<64, 128>(p, s);
}

}  // namespace locks
