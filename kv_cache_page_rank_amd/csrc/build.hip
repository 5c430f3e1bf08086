// Page summary builder (gist.science technical summary, section 2,
// Pagina-lokale Spectrale Decompositie: when a page is final its centred
// keys get a small eigendecomposition; the summary keeps the top-r
// eigenvectors and every token's coefficients; the centroid appears in the
// estimator of the same section).
//
// One 256-thread workgroup per (page, KV head), everything in LDS:
//  1. K (P x d) -> fp32, centroid mu, centred keys Kc.
//  2. Gram A = Kc Kc^T (P x P) on MFMA 16x16x4 fp32 (upper tiles, mirrored).
//  3. Cyclic two-sided Jacobi in round-robin (tournament) order: each round
//     rotates P/2 disjoint index pairs at once, A <- J^T A J, U <- U J.
//     Rotation angles follow the symmetric 2x2 Schur decomposition; sweeps
//     stop when a sweep rotates nothing or after kMaxSweeps.
//  4. Eigenvalues (diag A) ranked descending, ties by index; for the top r:
//     basis_k = Kc^T u / sqrt(lambda), re-orthonormalised by modified
//     Gram-Schmidt; coefficients are the coordinates coef[i][k] =
//     basis_k . (k_i - mu).  lambda <= 3e-5 lambda_max (or <= 0) is
//     numerically null and gives a zero basis row and coefficient column.
#include "device_common.hpp"
#include "launchers.hpp"

namespace locks {

namespace {

constexpr int kMaxSweeps = 20;
constexpr float kRelTol = 1e-6f;   // |a_pq| <= kRelTol sqrt(a_pp a_qq): already orthogonal
constexpr float kAbsTol = 2e-7f;   // |a_pq| <= kAbsTol trace(A): negligible coupling
constexpr float kNullTol = 3e-5f;  // lambda <= kNullTol lambda_max: numerically null

template <int P, int D, bool kBf16>
__global__ __launch_bounds__(256) void build_kernel(const BuildParams a) {
    constexpr int NPAIR = P / 2;
    constexpr int KP = D + 4;  // padded row of Kc
    constexpr int AP = P + 1;  // padded row of A and U
    __shared__ float kc[P][KP];
    __shared__ float A[P][AP];
    __shared__ float U[P][AP];
    __shared__ float mu_s[D];
    __shared__ float vs[16][D];
    __shared__ int rp[NPAIR], rq[NPAIR];
    __shared__ float rc[NPAIR], rs[NPAIR];
    __shared__ int rot_flag[2];
    __shared__ int slot[16];
    __shared__ float trace_s;

    // unit -> (b, page j, KV head g): every page of the table, or (refresh)
    // the refresh_pages pages from page_begin[b] on
    const int Hkv = a.num_kv_heads;
    const long u = blockIdx.x;
    const int g = (int)(u % Hkv);
    const int span = a.refresh_pages > 0 ? a.refresh_pages : a.max_pages;
    const int i = (int)((u / Hkv) % span);
    const int b = (int)(u / ((long)Hkv * span));
    int full = a.seq_lens[b] / P;
    full = full < 0 ? 0 : (full > a.max_pages ? a.max_pages : full);
    const int begin = a.page_begin ? a.page_begin[b] : 0;
    const int j = a.refresh_pages > 0 ? begin + i : i;
    if (j < begin || j < 0 || j >= full) return;  // uniform over the workgroup
    const int phys = a.block_table[(size_t)b * a.max_pages + j];
    if (phys < 0 || phys >= a.num_blocks) return;
    const int t = threadIdx.x;
    const int r = a.rank;
    const size_t unit = (size_t)phys * Hkv + g;

    // 1. keys -> LDS (fp32), centroid, centring
    if constexpr (kBf16) {
        const uint16_t* src = static_cast<const uint16_t*>(a.k) + unit * P * D;
        for (int i = t; i < P * D / 2; i += 256) {
            const uint32_t two = reinterpret_cast<const uint32_t*>(src)[i];
            const int row = (2 * i) / D, col = (2 * i) % D;
            kc[row][col] = __uint_as_float(two << 16);
            kc[row][col + 1] = __uint_as_float(two & 0xffff0000u);
        }
    } else {
        const float* src = static_cast<const float*>(a.k) + unit * P * D;
        for (int i = t; i < P * D; i += 256) kc[i / D][i % D] = src[i];
    }
    if (t == 0) {
        rot_flag[0] = 0;
        rot_flag[1] = 0;
    }
    __syncthreads();
    for (int d = t; d < D; d += 256) {
        float s = 0.f;
        for (int i = 0; i < P; ++i) s += kc[i][d];
        mu_s[d] = s / (float)P;
    }
    __syncthreads();
    for (int i = t; i < P * D; i += 256) kc[i / D][i % D] -= mu_s[i % D];
    for (int i = t; i < P * P; i += 256) U[i / P][i % P] = (i / P == i % P) ? 1.f : 0.f;
    __syncthreads();

    // 2. Gram on MFMA: tile (mi, ni), mi <= ni; A rows from block mi, B columns from block ni,
    //    contraction order d = 16*(s/4) + 4*(l/16) + s%4.
    {
        constexpr int NT = P / 16;
        constexpr int NTILES = NT * (NT + 1) / 2;
        const int wv = t >> 6, lane = t & 63, w = lane >> 4, c = lane & 15;
        for (int tile = wv; tile < NTILES; tile += 4) {
            int mi = 0, rem = tile;
            while (rem >= NT - mi) {
                rem -= NT - mi;
                ++mi;
            }
            const int ni = mi + rem;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int tq = 0; tq < D / 16; ++tq) {
                const f32x4 av = *reinterpret_cast<const f32x4*>(&kc[16 * mi + c][16 * tq + 4 * w]);
                const f32x4 bv = *reinterpret_cast<const f32x4*>(&kc[16 * ni + c][16 * tq + 4 * w]);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = mfma_16x16x4_f32(av[e], bv[e], acc);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = 16 * mi + 4 * w + v, col = 16 * ni + c;
                A[row][col] = acc[v];
                A[col][row] = acc[v];
            }
        }
    }
    __syncthreads();
    if (t == 0) {
        float tr = 0.f;
        for (int i = 0; i < P; ++i) tr += A[i][i];
        trace_s = tr;
    }
    __syncthreads();
    const float abs_tol = kAbsTol * trace_s;

    // 3. Jacobi sweeps
    for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
        for (int round = 0; round < P - 1; ++round) {
            if (t < NPAIR) {
                int p, q;
                if (t == 0) {
                    p = round;
                    q = P - 1;
                } else {
                    p = (round + t) % (P - 1);
                    q = (round - t + P - 1) % (P - 1);
                }
                if (p > q) {
                    const int x = p;
                    p = q;
                    q = x;
                }
                const float app = A[p][p], aqq = A[q][q], apq = A[p][q];
                float cs = 1.f, sn = 0.f;
                if (fabsf(apq) > kRelTol * sqrtf(fabsf(app * aqq)) && fabsf(apq) > abs_tol) {
                    const float zeta = (aqq - app) / (2.f * apq);
                    const float tn = (zeta >= 0.f ? 1.f : -1.f) / (fabsf(zeta) + sqrtf(1.f + zeta * zeta));
                    cs = 1.f / sqrtf(1.f + tn * tn);
                    sn = tn * cs;
                    rot_flag[sweep & 1] = 1;
                }
                rp[t] = p;
                rq[t] = q;
                rc[t] = cs;
                rs[t] = sn;
            }
            __syncthreads();
            if (round == 0 && t == 0) rot_flag[(sweep + 1) & 1] = 0;
            // A <- J^T A J on 2x2 blocks (pair a rows, pair bb columns)
            for (int bi = t; bi < NPAIR * NPAIR; bi += 256) {
                const int pa_i = bi / NPAIR, pb_i = bi % NPAIR;
                const float ca = rc[pa_i], sa = rs[pa_i], cb = rc[pb_i], sb = rs[pb_i];
                if (sa == 0.f && sb == 0.f) continue;
                const int pa = rp[pa_i], qa = rq[pa_i], pb = rp[pb_i], qb = rq[pb_i];
                const float x = A[pa][pb], y = A[pa][qb], z = A[qa][pb], wv = A[qa][qb];
                const float x1 = x * cb - y * sb, y1 = x * sb + y * cb;
                const float z1 = z * cb - wv * sb, w1 = z * sb + wv * cb;
                A[pa][pb] = ca * x1 - sa * z1;
                A[qa][qb] = sa * y1 + ca * w1;
                if (pa_i == pb_i) {
                    A[pa][qb] = 0.f;
                    A[qa][pb] = 0.f;
                } else {
                    A[pa][qb] = ca * y1 - sa * w1;
                    A[qa][pb] = sa * x1 + ca * z1;
                }
            }
            // U <- U J
            for (int ui = t; ui < P * NPAIR; ui += 256) {
                const int row = ui / NPAIR, pr = ui % NPAIR;
                const float cs = rc[pr], sn = rs[pr];
                if (sn == 0.f) continue;
                const int p = rp[pr], q = rq[pr];
                const float up = U[row][p], uq = U[row][q];
                U[row][p] = cs * up - sn * uq;
                U[row][q] = sn * up + cs * uq;
            }
            __syncthreads();
        }
        if (rot_flag[sweep & 1] == 0) break;  // same value for every thread
    }

    // 4. rank eigenvalues, emit the top r
    if (t < P) {
        const float lam = A[t][t];
        int rank = 0;
        for (int i = 0; i < P; ++i) {
            const float li = A[i][i];
            rank += (li > lam || (li == lam && i < t)) ? 1 : 0;
        }
        if (rank < r) slot[rank] = t;
    }
    __syncthreads();
    const float lam_max = A[slot[0]][slot[0]];
    // basis rows basis_k = Kc^T u_k / sqrt(lambda_k) (zero for null directions)
    for (int i = t; i < r * D; i += 256) {
        const int k = i / D, d = i % D;
        const int e = slot[k];
        const float lam = A[e][e];
        float s = 0.f;
        if (lam > 0.f && lam > kNullTol * lam_max) {
            for (int tok = 0; tok < P; ++tok) s += kc[tok][d] * U[tok][e];
            s /= sqrtf(lam);
        }
        vs[k][d] = s;
    }
    __syncthreads();
    // Re-orthonormalise the rows (modified Gram-Schmidt, two passes, largest
    // eigenvalue first): the fp32 Gram squares the conditioning, so rows of
    // small-eigenvalue directions are orthonormal only to ~1e-4 otherwise.
    if (t < kWave) {
        constexpr int DL = D / kWave;  // dims per lane
        for (int k = 0; k < r; ++k) {
            float x[DL];
            float nrm2 = 0.f;
#pragma unroll
            for (int e = 0; e < DL; ++e) {
                x[e] = vs[k][t + kWave * e];
                nrm2 += x[e] * x[e];
            }
            if (wave_sum(nrm2) == 0.f) continue;  // null direction stays zero
            for (int pass = 0; pass < 2; ++pass) {
                for (int jr = 0; jr < k; ++jr) {
                    float dp = 0.f;
#pragma unroll
                    for (int e = 0; e < DL; ++e) dp += x[e] * vs[jr][t + kWave * e];
                    dp = wave_sum(dp);
#pragma unroll
                    for (int e = 0; e < DL; ++e) x[e] -= dp * vs[jr][t + kWave * e];
                }
            }
            nrm2 = 0.f;
#pragma unroll
            for (int e = 0; e < DL; ++e) nrm2 += x[e] * x[e];
            const float inv = 1.f / sqrtf(wave_sum(nrm2));
#pragma unroll
            for (int e = 0; e < DL; ++e) vs[k][t + kWave * e] = x[e] * inv;
        }
    }
    __syncthreads();
    // outputs: centroid, basis, coefficients = coordinates Kc V^T, stored as
    // fp32 or rounded to bf16 (nearest even)
    auto put = [&](void* base, size_t idx, float v) {
        if (a.out_bf16)
            static_cast<uint16_t*>(base)[idx] = f32_to_bf16_bits(v);
        else
            static_cast<float*>(base)[idx] = v;
    };
    const size_t mu0 = unit * D, basis0 = unit * (size_t)r * D, coef0 = unit * (size_t)P * r;
    for (int d = t; d < D; d += 256) put(a.mu, mu0 + d, mu_s[d]);
    for (int i = t; i < r * D; i += 256) put(a.basis, basis0 + i, vs[i / D][i % D]);
    for (int i = t; i < P * r; i += 256) {
        const int tok = i / r, k = i % r;
        float s = 0.f;
        for (int d = 0; d < D; ++d) s += kc[tok][d] * vs[k][d];
        put(a.coef, coef0 + i, s);
    }
}

template <int P, int D>
hipError_t launch_pd(const BuildParams& p, hipStream_t s) {
    const long units =
        (long)p.batch * (p.refresh_pages > 0 ? p.refresh_pages : p.max_pages) * p.num_kv_heads;
    if (units == 0) return hipSuccess;
    if (p.bf16)
        hipLaunchKernelGGL((build_kernel<P, D, true>), dim3((unsigned)units), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((build_kernel<P, D, false>), dim3((unsigned)units), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

bool build_supported(int page_size, int head_dim, int rank) {
    return (page_size == 16 || page_size == 64) && (head_dim == 64 || head_dim == 128) &&
           rank >= 1 && rank <= 16 && rank <= page_size && rank <= head_dim;
}

hipError_t launch_build(const BuildParams& p, hipStream_t s) {
    if (p.page_size == 16 && p.head_dim == 64) return launch_pd<16, 64>(p, s);
    if (p.page_size == 16 && p.head_dim == 128) return launch_pd<16, 128>(p, s);
    if (p.page_size == 64 && p.head_dim == 64) return launch_pd<64, 64>(p, s);
    return launch_pd<64, 128>(p, s);
}

}  // namespace locks
