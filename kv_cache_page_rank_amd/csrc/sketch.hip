// Shared-basis sketch, the ablation baseline (technical summary, section 3:
// a query-independent projection shared by every page is blind to
// page-specific directions; the abstract contrasts the page-local summary
// with fixed sketches).  Given one rank-rho basis per KV head, every full
// page keeps its centroid and its tokens' coordinates in that basis; the
// result is written in the page-summary layout (the basis copied to each
// block) so the same scan scores it with the same estimator.
//
// One 256-thread workgroup per (page, KV head): keys -> LDS (fp32), centroid,
// centring, then coef[i][k] = (k_i - mu) . basis_k over d.
#include "device_common.hpp"
#include "launchers.hpp"

namespace locks {

namespace {

constexpr int kSketchThreads = 256;

template <int P, int D, bool kBf16>
__global__ __launch_bounds__(kSketchThreads) void sketch_kernel(const BuildParams a,
                                                                const float* shared_basis) {
    constexpr int KP = D + 4;
    __shared__ float kc[P][KP];
    __shared__ float vb[16][D];
    __shared__ float mu_s[D];
    const int Hkv = a.num_kv_heads;
    const long u = blockIdx.x;
    const int g = (int)(u % Hkv);
    const int j = (int)((u / Hkv) % a.max_pages);
    const int b = (int)(u / ((long)Hkv * a.max_pages));
    int full = a.seq_lens[b] / P;
    full = full < 0 ? 0 : (full > a.max_pages ? a.max_pages : full);
    const int begin = a.page_begin ? a.page_begin[b] : 0;
    if (j < begin || j >= full) return;  // uniform over the workgroup
    const int phys = a.block_table[(size_t)b * a.max_pages + j];
    if (phys < 0 || phys >= a.num_blocks) return;
    const int t = threadIdx.x, r = a.rank;
    const size_t unit = (size_t)phys * Hkv + g;

    if constexpr (kBf16) {
        const uint16_t* src = static_cast<const uint16_t*>(a.k) + unit * P * D;
        for (int i = t; i < P * D; i += kSketchThreads) kc[i / D][i % D] = bf16_bits_to_f32(src[i]);
    } else {
        const float* src = static_cast<const float*>(a.k) + unit * P * D;
        for (int i = t; i < P * D; i += kSketchThreads) kc[i / D][i % D] = src[i];
    }
    const float* V = shared_basis + (size_t)g * r * D;
    for (int i = t; i < r * D; i += kSketchThreads) vb[i / D][i % D] = V[i];
    __syncthreads();
    for (int d = t; d < D; d += kSketchThreads) {
        float s = 0.f;
        for (int i = 0; i < P; ++i) s += kc[i][d];
        mu_s[d] = s / (float)P;
    }
    __syncthreads();
    for (int i = t; i < P * D; i += kSketchThreads) kc[i / D][i % D] -= mu_s[i % D];
    __syncthreads();
    float* mu = static_cast<float*>(a.mu) + unit * D;
    float* basis = static_cast<float*>(a.basis) + unit * (size_t)r * D;
    float* coef = static_cast<float*>(a.coef) + unit * (size_t)P * r;
    for (int d = t; d < D; d += kSketchThreads) mu[d] = mu_s[d];
    for (int i = t; i < r * D; i += kSketchThreads) basis[i] = vb[i / D][i % D];
    for (int i = t; i < P * r; i += kSketchThreads) {
        const int tok = i / r, k = i % r;
        float s = 0.f;
        for (int d = 0; d < D; ++d) s += kc[tok][d] * vb[k][d];
        coef[i] = s;
    }
}

template <int P, int D>
hipError_t launch_pd(const BuildParams& p, const float* basis, hipStream_t s) {
    const long units = (long)p.batch * p.max_pages * p.num_kv_heads;
    if (units == 0) return hipSuccess;
    if (p.bf16)
        hipLaunchKernelGGL((sketch_kernel<P, D, true>), dim3((unsigned)units), dim3(kSketchThreads),
                           0, s, p, basis);
    else
        hipLaunchKernelGGL((sketch_kernel<P, D, false>), dim3((unsigned)units),
                           dim3(kSketchThreads), 0, s, p, basis);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sketch(const BuildParams& p, const float* shared_basis, hipStream_t s) {
    if (p.page_size == 16 && p.head_dim == 64) return launch_pd<16, 64>(p, shared_basis, s);
    if (p.page_size == 16 && p.head_dim == 128) return launch_pd<16, 128>(p, shared_basis, s);
    if (p.page_size == 64 && p.head_dim == 64) return launch_pd<64, 64>(p, shared_basis, s);
    return launch_pd<64, 128>(p, shared_basis, s);
}

}  // namespace locks
