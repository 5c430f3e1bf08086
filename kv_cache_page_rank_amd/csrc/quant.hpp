// Summary quantiser (technical summary, section 2, Kwantisatie: the basis
// is stored in int4, coefficients and centroid in int8).  Shared by the
// summary builder (quantised output) and the stand-alone quantise kernel, so
// both emit the same codes.  Per vector (the centroid, each basis row, each
// coefficient column): scale = max|x| / Q by IEEE float division (HIP's
// default division is correctly rounded), code = round-half-even(x / scale)
// clamped to [-Q, Q], Q = 127 (int8) or 7 (int4); a zero vector keeps scale
// 0 and codes 0.  int4 codes: element 2t in the low nibble of byte t.
#pragma once

#include "device_common.hpp"

namespace locks {

constexpr int kQ8 = 127;
constexpr int kQ4 = 7;

__device__ __forceinline__ int quant_code(float x, float s, int qmax) {
    if (!(s > 0.f)) return 0;
    const int c = (int)rintf(x / s);
    return c > qmax ? qmax : (c < -qmax ? -qmax : c);
}

// One unit's codes and scales from fp32 values in LDS: mu [D]; basis rows k
// at basis[k * bstride .. + D); coefficients coef[tok * cstride + k].
// Every thread of the workgroup (NT threads) calls it; amax and qs are LDS
// scratch of 1 + 2 * 16 floats.  Global outputs of this unit: mu_q [D],
// basis_q [r][D/2], coef_q [P][r], scales [1 + 2r].
template <int P, int D, int NT>
__device__ __forceinline__ void quantize_unit(const float* mu, const float* basis, int bstride,
                                              const float* coef, int cstride, int r,
                                              int8_t* mu_q, uint8_t* basis_q, int8_t* coef_q,
                                              float* scales, float* amax, float* qs, int t) {
    const int nv = 1 + 2 * r;
    const int wave = t / kWave, lane = t % kWave;
    for (int v = wave; v < nv; v += NT / kWave) {
        float m = 0.f;
        if (v == 0) {
            for (int i = lane; i < D; i += kWave) m = fmaxf(m, fabsf(mu[i]));
        } else if (v <= r) {
            for (int i = lane; i < D; i += kWave) m = fmaxf(m, fabsf(basis[(v - 1) * bstride + i]));
        } else {
            for (int i = lane; i < P; i += kWave) m = fmaxf(m, fabsf(coef[i * cstride + (v - 1 - r)]));
        }
        m = wave_max(m);
        if (lane == 0) amax[v] = m;
    }
    __syncthreads();
    if (t < nv) {
        const float s = amax[t] / (float)(t >= 1 && t <= r ? kQ4 : kQ8);
        qs[t] = s;
        scales[t] = s;
    }
    __syncthreads();
    for (int i = t; i < D; i += NT) mu_q[i] = (int8_t)quant_code(mu[i], qs[0], kQ8);
    for (int i = t; i < r * (D / 2); i += NT) {
        const int k = i / (D / 2), e = 2 * (i % (D / 2));
        const int lo = quant_code(basis[k * bstride + e], qs[1 + k], kQ4);
        const int hi = quant_code(basis[k * bstride + e + 1], qs[1 + k], kQ4);
        basis_q[i] = (uint8_t)((lo & 15) | ((hi & 15) << 4));
    }
    for (int i = t; i < P * r; i += NT) {
        const int tok = i / r, k = i % r;
        coef_q[i] = (int8_t)quant_code(coef[tok * cstride + k], qs[1 + r + k], kQ8);
    }
}

}  // namespace locks
