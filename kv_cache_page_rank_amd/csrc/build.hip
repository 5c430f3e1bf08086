// Page summary builder (gist.science technical summary, section 2,
// Pagina-lokale Spectrale Decompositie: when a page is final its centred
// keys get a small eigendecomposition; the summary keeps the top-r
// eigenvectors and every token's coefficients; the centroid appears in the
// estimator of the same section).
//
// One workgroup per (page, KV head) (13 waves at P = 64, 3 at P = 16),
// everything in LDS:
//  1. K (P x d) -> fp32, centroid mu, centred keys Kc.
//  2. Gram A = Kc Kc^T (P x P) on MFMA 16x16x4 fp32 (upper tiles).
//  3. Cyclic two-sided Jacobi in round-robin (tournament) order: each round
//     rotates P/2 disjoint index pairs at once, A <- J^T A J, U <- U J.
//     Rotation angles follow the symmetric 2x2 Schur decomposition; sweeps
//     stop once no pair of the matrix couples any more (checked over the
//     whole matrix after each sweep, which spares the last, idle sweep) or
//     after kMaxSweeps.  One polishing sweep follows with a much tighter
//     tolerance and no absolute floor beyond what keeps the angle finite: the
//     stopping rule's floor (2e-7 of the trace) lets couplings of ~1e-5
//     between the small eigenvalues stand, which turns the rank-r subspace
//     by ~1e-4 whenever the eigenvalues on either side of the cut lie close;
//     one more sweep, converging quadratically, removes them (the polished
//     basis reconstructs logits to ~1e-5 of the double-precision summary on
//     the 128-dimensional pages of the workloads, against ~3e-4 without).
//     A is kept in position space, where a round's pairs
//     are always adjacent positions and a fixed permutation moves every
//     index between rounds, so each thread owns one 2x2 block with read and
//     write slots fixed for the whole kernel (a round is a few loads, eight
//     multiply-adds and four stores); only the upper triangle is kept.  U's
//     columns move the same way; its updates trail by a round and run on
//     every other wave while wave 0 computes the next round's rotations.  U's buffers take Kc's place
//     during the sweeps, and Kc is read again afterwards.
//  4. Eigenvalues (diag A) ranked descending, ties by index; for the top r:
//     basis_k = Kc^T u / sqrt(lambda), re-orthonormalised by modified
//     Gram-Schmidt.  lambda <= 3e-6 lambda_max (or <= 0) is numerically null
//     and gives a zero basis row and coefficient column.
//  5. Two steps of subspace iteration on the top r rows, applied through Kc
//     itself: Y = Kc V^T (P x r), then V^T <- Kc^T Y, re-orthonormalised.  The
//     Gram squares the conditioning: its fp32 rounding (~1e-7 lambda_max)
//     moves the rank-r subspace by that over lambda_r - lambda_{r+1}, which
//     is large when the page's small eigenvalues are small in absolute terms
//     (pages with little noise).  Products with Kc carry rounding of only
//     ~1e-7 sigma_1 sigma_k, and each step also shrinks the components
//     outside the subspace by lambda_{r+1} / lambda_r, so the subspace ends
//     near the accuracy of an SVD of Kc.
//  6. Coefficients are the coordinates coef[i][k] = basis_k . (k_i - mu).
#include "device_common.hpp"
#include "launchers.hpp"
#include "quant.hpp"

namespace locks {

namespace {

constexpr int kMaxSweeps = 20;
constexpr float kRelTol = 1e-6f;   // |a_pq| <= kRelTol sqrt(a_pp a_qq): already orthogonal
constexpr float kAbsTol = 2e-7f;   // |a_pq| <= kAbsTol trace(A): negligible coupling
constexpr float kPolishRelTol = 1e-7f;  // the polishing sweep's relative tolerance
constexpr float kPolishAbsTol = 1e-12f; // and its floor (keeps zeta finite, see jacobi_angle)
constexpr float kNullTol = 3e-6f;  // lambda <= kNullTol lambda_max: numerically null
constexpr int kRefineSteps = 2;    // subspace-iteration steps through Kc

// Waves: 0 (rotations, diagonal blocks), 1..NOFFW (off-diagonal blocks of
// A), then the U waves (eight row updates per lane and round at P = 64).
template <int P>
constexpr int build_off_waves() {
    return ((P / 2) * (P / 2 - 1) / 2 + kWave - 1) / kWave;
}
template <int P>
constexpr int build_u_waves() {
    return P * (P / 2) >= 8 * kWave ? P * (P / 2) / (8 * kWave) : 1;
}
template <int P>
constexpr int build_threads() {
    return kWave * (1 + build_off_waves<P>() + build_u_waves<P>());
}

// Pair i of round rd: (rd, P-1) for i = 0, else ((rd + i) mod (P-1),
// (rd - i) mod (P-1)).  Plain arithmetic: with rd and i known at compile
// time both fold to constants.
template <int P>
__device__ constexpr int pair_a(int rd, int i) {
    return i == 0 ? rd : (rd + i >= P - 1 ? rd + i - (P - 1) : rd + i);
}
template <int P>
__device__ constexpr int pair_b(int rd, int i) {
    return i == 0 ? P - 1 : (rd - i + (P - 1) >= P - 1 ? rd - i : rd - i + (P - 1));
}

// Position space.  In round rd, pair i sits at positions (2i, 2i+1): its
// first index pair_a at 2i, its second pair_b at 2i+1.  Between rounds every
// index moves by the same permutation sigma (the first indices shift down a
// pair, the second ones up, with turns at both ends and P-1 fixed), and after
// P-1 rounds the layout is back to pos0.
template <int P>
__device__ constexpr int pos0(int x) {
    return x == 0 ? 0 : x == P - 1 ? 1 : x < P / 2 ? 2 * x : 2 * (P - 1 - x) + 1;
}
template <int P>
__device__ constexpr int sigma(int pos) {
    return pos == 0   ? 3
           : pos == 1 ? 1
           : pos == 2 ? 0
           : (pos & 1) == 0 ? pos - 2
           : pos == P - 1   ? P - 2
                            : pos + 2;
}

// Pair (p, q) still couples: |a_pq| above rel_tol sqrt(|a_pp a_qq|) (compared
// squared, rel2 = rel_tol^2) and above the absolute floor.
__device__ __forceinline__ bool couples(float app, float aqq, float apq, float abs_tol,
                                        float rel2 = kRelTol * kRelTol) {
    return apq * apq > rel2 * fabsf(app * aqq) && fabsf(apq) > abs_tol;
}

// Rotation (cos, sin) that zeroes a_pq of the symmetric 2x2 block: with
// zeta = (a_qq - a_pp) / (2 a_pq), tan = sign(zeta) / (|zeta| + sqrt(1 + zeta^2))
// (the smaller of the two angles).  Hardware reciprocal / square root (1 ulp)
// keep the dependent chain short; cos^2 + sin^2 = 1 holds to a few ulp, which
// is all the sweep needs.  |a_pq| > the absolute floor >= trace * kAbsTol
// bounds |zeta| (diagonal >= 0, so |a_qq - a_pp| <= trace): no overflow.
__device__ __forceinline__ void jacobi_angle(float app, float aqq, float apq, float& cs,
                                             float& sn, float& tn) {
    const float zeta = (aqq - app) * __builtin_amdgcn_rcpf(2.f * apq);
    const float az = fabsf(zeta);
    tn = __builtin_amdgcn_rcpf(az + __builtin_amdgcn_sqrtf(1.f + az * az));
    tn = zeta >= 0.f ? tn : -tn;
    cs = __builtin_amdgcn_rsqf(1.f + tn * tn);
    sn = tn * cs;
}

template <int P, int D, bool kBf16>
__global__ __launch_bounds__(build_threads<P>()) void build_kernel(const BuildParams a) {
    constexpr int NT = build_threads<P>();
    constexpr int NPAIR = P / 2;
    constexpr int NOFF = NPAIR * (NPAIR - 1) / 2;           // off-diagonal 2x2 blocks
    constexpr int NOFFW = build_off_waves<P>();             // their waves
    constexpr int UW0 = NOFFW + 1;                          // first U wave
    // U's updates run in the rotation phase, when every wave but wave 0 is
    // otherwise idle: all of them share the rows (2-3 per thread at P = 64)
    constexpr int NUT = NT - kWave;                         // threads rotating U
    constexpr int USTEP = NUT / NPAIR;                      // row stride of a U thread
    constexpr int UROWS = (P + USTEP - 1) / USTEP;          // rows per U thread, at most
    static_assert(NPAIR <= kWave && NUT % NPAIR == 0, "wave roles");
    constexpr int KP = D + 4;   // padded row of Kc
    constexpr int S = P + 2;    // row of a position-space matrix (even: 8-byte pairs)
    constexpr int UP = P + 1;   // padded row of U
    // the Jacobi's two position-space buffers of A; afterwards U and the basis rows
    // (and, for quantised output, the coefficients)
    constexpr int JB = 2 * P * S > P * UP + 16 * D + 16 * P ? 2 * P * S : P * UP + 16 * D + 16 * P;
    // Kc; during the sweeps (Kc idle) the two position-space buffers of U
    constexpr int KB = P * KP > 2 * P * S ? P * KP : 2 * P * S;
    __shared__ __attribute__((aligned(16))) float kbuf[KB];
    __shared__ __attribute__((aligned(16))) float jbuf[JB];
    float (*const kc)[KP] = reinterpret_cast<float (*)[KP]>(kbuf);
    __shared__ float mu_s[D];
    __shared__ float lam_s[P];
    __shared__ __attribute__((aligned(16))) f32x2 ring[2][NPAIR];  // (cos, sin), two rounds
    __shared__ int more[2];           // a sweep left a coupled pair (by sweep parity)
    __shared__ int slot[16];
    __shared__ float trace_s;
    __shared__ float q_amax[1 + 2 * 16], q_s[1 + 2 * 16];  // quantiser scratch
    float (*const U)[UP] = reinterpret_cast<float (*)[UP]>(jbuf);
    float (*const vs)[D] = reinterpret_cast<float (*)[D]>(jbuf + P * UP);
    // canonical (upper) slot of position-space entry (x, y)
    auto at = [](int x, int y) { return x < y ? x * S + y : y * S + x; };

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
    auto load_keys = [&]() {
        if constexpr (kBf16) {
            const uint16_t* src = static_cast<const uint16_t*>(a.k) + unit * P * D;
            for (int i = t; i < P * D / 2; i += NT) {
                const uint32_t two = reinterpret_cast<const uint32_t*>(src)[i];
                const int row = (2 * i) / D, col = (2 * i) % D;
                kc[row][col] = __uint_as_float(two << 16);
                kc[row][col + 1] = __uint_as_float(two & 0xffff0000u);
            }
        } else {
            const float* src = static_cast<const float*>(a.k) + unit * P * D;
            for (int i = t; i < P * D; i += NT) kc[i / D][i % D] = src[i];
        }
    };
    load_keys();
    if (t == 0) {
        more[0] = 0;
        more[1] = 0;
    }
    __syncthreads();
    for (int d = t; d < D; d += NT) {
        float s = 0.f;
        for (int i = 0; i < P; ++i) s += kc[i][d];
        mu_s[d] = s / (float)P;
    }
    __syncthreads();
    for (int i = t; i < P * D; i += NT) kc[i / D][i % D] -= mu_s[i % D];
    __syncthreads();

    // 2. Gram on MFMA: tile (mi, ni), mi <= ni; A rows from block mi, B columns from block ni,
    //    contraction order d = 16*(s/4) + 4*(l/16) + s%4.
    {
        constexpr int NB16 = P / 16;
        constexpr int NTILES = NB16 * (NB16 + 1) / 2;
        const int wv = t >> 6, lane = t & 63, w = lane >> 4, c = lane & 15;
        for (int tile = wv; tile < NTILES; tile += NT / kWave) {
            int mi = 0, rem = tile;
            while (rem >= NB16 - mi) {
                rem -= NB16 - mi;
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
                if (row <= col) jbuf[at(pos0<P>(row), pos0<P>(col))] = acc[v];
            }
        }
    }
    __syncthreads();
    if (t == 0) {
        float tr = 0.f;
        for (int i = 0; i < P; ++i) tr += jbuf[i * S + i];
        trace_s = tr;
    }
    __syncthreads();
    const float abs_tol = fmaxf(kAbsTol * trace_s, 1e-30f);
    const float polish_abs_tol = fmaxf(kPolishAbsTol * trace_s, 1e-30f);

    // 3. Jacobi sweeps in position space (pair i at positions 2i, 2i+1),
    //    ping-ponging between two buffers.  Every thread's read and write
    //    slots are fixed for the whole kernel: a round rotates its block and
    //    stores it where sigma puts it.  Wave 0 lane i owns diagonal block i
    //    of A and computes pair i's rotation; waves 1..NOFFW own the
    //    off-diagonal blocks (upper triangle only); the U waves rotate column
    //    pairs of U (whose columns move by sigma like A's), a round behind,
    //    while the next round's rotations are being computed.  Two barriers
    //    per round (rotations ready; blocks moved), one more per sweep
    //    (convergence).
    const int wave = __builtin_amdgcn_readfirstlane(t / kWave);  // wave-uniform role
    float* const ubuf = kbuf;  // U's two buffers while Kc is idle
    for (int e = t; e < P * P; e += NT) {
        const int row = e / P, col = e % P;
        ubuf[row * S + pos0<P>(col)] = row == col ? 1.f : 0.f;
    }
    // this thread's block of A: wave 0 -> diagonal block t; else off-diagonal
    // block (ba, bb), ba < bb, numbered row by row
    int ba = 0, bb = 0;
    if (wave == 0) {
        ba = bb = t;
    } else if (wave < UW0) {
        int rem = t - kWave;
        while (rem >= NPAIR - 1 - ba && ba < NPAIR - 1) {
            rem -= NPAIR - 1 - ba;
            ++ba;
        }
        bb = ba + 1 + rem;
    }
    const bool diag = wave == 0 && t < NPAIR;
    const bool offd = wave > 0 && wave < UW0 && t - kWave < NOFF;
    const int r0 = 2 * ba, r1 = 2 * ba + 1, c0 = 2 * bb, c1 = 2 * bb + 1;
    const int s0 = sigma<P>(r0), s1 = sigma<P>(r1), e0 = sigma<P>(c0), e1 = sigma<P>(c1);
    const int src0 = r0 * S + c0, src1 = r1 * S + c0;  // 8-byte row pairs (upper: r < c)
    const int d00 = at(s0, e0), d01 = at(s0, e1), d10 = at(s1, e0), d11 = at(s1, e1);
    // U thread: column pair ui, rows urow + USTEP * m below P
    const bool uthr = wave >= 1;
    const int ut = t - kWave;
    const int ui = uthr ? ut % NPAIR : 0, urow = uthr ? ut / NPAIR : 0;
    const int usrc = urow * S + 2 * ui;
    const int ud0 = urow * S + sigma<P>(2 * ui), ud1 = urow * S + sigma<P>(2 * ui + 1);
    // U <- U J of round k (rotations in ring[k & 1]), buffer k & 1 -> the other
    auto rotate_u = [&](int k) {
        const f32x2 rot = ring[k & 1][ui];
        const float* cur = ubuf + (k & 1) * (P * S);
        float* nxt = ubuf + ((k + 1) & 1) * (P * S);
#pragma unroll
        for (int m = 0; m < UROWS; ++m) {
            if (urow + m * USTEP < P) {
                const f32x2 v = *reinterpret_cast<const f32x2*>(cur + usrc + m * USTEP * S);
                nxt[ud0 + m * USTEP * S] = rot[0] * v[0] - rot[1] * v[1];
                nxt[ud1 + m * USTEP * S] = rot[1] * v[0] + rot[0] * v[1];
            }
        }
    };
    __syncthreads();
    int rounds = 0;
    // rotation test of the current sweep: the stopping rule's, then the
    // polishing sweep's
    float rot_abs = abs_tol, rot_rel2 = kRelTol * kRelTol;
    bool polishing = false;
    for (int sweep = 0;; ++sweep) {
        for (int rd = 0; rd < P - 1; ++rd, ++rounds) {
            const float* cur = jbuf + (rounds & 1) * (P * S);
            float* nxt = jbuf + ((rounds + 1) & 1) * (P * S);
            // phase (i): the round's rotations; a diagonal block moves at once
            // (nothing reads the other buffer in this round); U catches up
            if (diag) {
                const float app = cur[r0 * S + r0], aqq = cur[r1 * S + r1];
                const float apq = cur[r0 * S + r1];
                float cs = 1.f, sn = 0.f, tn = 0.f;
                const bool rot = couples(app, aqq, apq, rot_abs, rot_rel2);
                if (rot) jacobi_angle(app, aqq, apq, cs, sn, tn);
                ring[rounds & 1][t] = f32x2{cs, sn};
                nxt[s0 * S + s0] = app - tn * apq;
                nxt[s1 * S + s1] = aqq + tn * apq;
                nxt[d01] = rot ? 0.f : apq;
            }
            if (uthr && rounds > 0) rotate_u(rounds - 1);
            __syncthreads();
            // the flag of the next sweep is cleared once every thread has read it
            if (rd == 0 && t == 0) more[(sweep + 1) & 1] = 0;
            // phase (ii): off-diagonal block <- J_a^T block J_b, moved by sigma
            if (offd) {
                const f32x2 ra = ring[rounds & 1][ba], rb = ring[rounds & 1][bb];
                const f32x2 top = *reinterpret_cast<const f32x2*>(cur + src0);
                const f32x2 bot = *reinterpret_cast<const f32x2*>(cur + src1);
                const float ca = ra[0], sa = ra[1], cb = rb[0], sb = rb[1];
                const float x1 = top[0] * cb - top[1] * sb, y1 = top[0] * sb + top[1] * cb;
                const float z1 = bot[0] * cb - bot[1] * sb, w1 = bot[0] * sb + bot[1] * cb;
                nxt[d00] = ca * x1 - sa * z1;
                nxt[d01] = ca * y1 - sa * w1;
                nxt[d10] = sa * x1 + ca * z1;
                nxt[d11] = sa * y1 + ca * w1;
            }
            __syncthreads();
        }
        if (polishing) break;  // the polishing sweep is the last
        // Converged when no pair of the matrix couples any more: the next
        // sweep would rotate nothing by the stopping rule; the polishing
        // sweep runs instead.
        const float* fin = jbuf + (rounds & 1) * (P * S);
        bool coupled = false;
        for (int e = t; e < P * P; e += NT) {
            const int x = e / P, y = e % P;
            if (x < y) coupled |= couples(fin[x * S + x], fin[y * S + y], fin[x * S + y], abs_tol);
        }
        if (coupled) more[sweep & 1] = 1;
        __syncthreads();
        if (more[sweep & 1] == 0 || sweep + 1 >= kMaxSweeps) {  // same for every thread
            polishing = true;
            rot_abs = polish_abs_tol;
            rot_rel2 = kPolishRelTol * kPolishRelTol;
        }
    }
    if (uthr && rounds > 0) rotate_u(rounds - 1);  // the last round's rotations
    // sweeps end with the layout back at pos0: eigenvalue of index x
    {
        const float* fin = jbuf + (rounds & 1) * (P * S);
        if (t < P) lam_s[t] = fin[pos0<P>(t) * S + pos0<P>(t)];
    }
    __syncthreads();
    // U to index space (over A's buffers), then Kc again
    {
        const float* uf = ubuf + (rounds & 1) * (P * S);
        for (int e = t; e < P * P; e += NT) {
            const int row = e / P, col = e % P;
            U[row][col] = uf[row * S + pos0<P>(col)];
        }
    }
    __syncthreads();
    load_keys();
    __syncthreads();
    for (int i = t; i < P * D; i += NT) kc[i / D][i % D] -= mu_s[i % D];
    __syncthreads();

    // 4. rank eigenvalues, emit the top r
    if (t < P) {
        const float lam = lam_s[t];
        int rank = 0;
        for (int i = 0; i < P; ++i) {
            const float li = lam_s[i];
            rank += (li > lam || (li == lam && i < t)) ? 1 : 0;
        }
        if (rank < r) slot[rank] = t;
    }
    __syncthreads();
    const float lam_max = lam_s[slot[0]];
    // basis rows basis_k = Kc^T u_k / sqrt(lambda_k) (zero for null directions)
    for (int i = t; i < r * D; i += NT) {
        const int k = i / D, d = i % D;
        const int e = slot[k];
        const float lam = lam_s[e];
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
    auto orthonormalise_rows = [&]() {
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
    };
    orthonormalise_rows();
    // 5. subspace iteration through Kc: Y = Kc V^T, V^T <- Kc^T Y, orthonormalised
    {
        float (*const ys)[16] = reinterpret_cast<float (*)[16]>(jbuf + P * UP + 16 * D);  // [P][r]
        for (int step = 0; step < kRefineSteps; ++step) {
            for (int i = t; i < P * r; i += NT) {
                const int k = i / P, tok = i % P;  // a wave shares one basis row
                float s = 0.f;
#pragma unroll 8
                for (int d = 0; d < D; d += 4) {
                    const f32x4 x = *reinterpret_cast<const f32x4*>(&kc[tok][d]);
                    const f32x4 v = *reinterpret_cast<const f32x4*>(&vs[k][d]);
                    s += x[0] * v[0] + x[1] * v[1] + x[2] * v[2] + x[3] * v[3];
                }
                ys[tok][k] = s;
            }
            __syncthreads();
            for (int i = t; i < r * D; i += NT) {
                const int k = i / D, d = i % D;
                float s = 0.f;
                for (int tok = 0; tok < P; ++tok) s += kc[tok][d] * ys[tok][k];
                vs[k][d] = s;
            }
            __syncthreads();
            orthonormalise_rows();
        }
    }
    // outputs: centroid, basis, coefficients = coordinates Kc V^T, stored as
    // fp32, rounded to bf16 (nearest even), or as int8 / int4 codes
    if (a.out_dtype == kSummQ8Q4) {
        float* cs = jbuf + P * UP + 16 * D;  // [P][r] coefficients, after U and the basis rows
        for (int i = t; i < P * r; i += NT) {
            const int tok = i / r, k = i % r;
            float s = 0.f;
            for (int d = 0; d < D; ++d) s += kc[tok][d] * vs[k][d];
            cs[i] = s;
        }
        __syncthreads();
        quantize_unit<P, D, NT>(mu_s, &vs[0][0], D, cs, r, r,
                                static_cast<int8_t*>(a.mu) + unit * D,
                                static_cast<uint8_t*>(a.basis) + unit * (size_t)r * (D / 2),
                                static_cast<int8_t*>(a.coef) + unit * (size_t)P * r,
                                a.scales + unit * (size_t)(1 + 2 * r), q_amax, q_s, t);
        return;
    }
    auto put = [&](void* base, size_t idx, float v) {
        if (a.out_dtype == kSummBF16)
            static_cast<uint16_t*>(base)[idx] = f32_to_bf16_bits(v);
        else
            static_cast<float*>(base)[idx] = v;
    };
    const size_t mu0 = unit * D, basis0 = unit * (size_t)r * D, coef0 = unit * (size_t)P * r;
    for (int d = t; d < D; d += NT) put(a.mu, mu0 + d, mu_s[d]);
    for (int i = t; i < r * D; i += NT) put(a.basis, basis0 + i, vs[i / D][i % D]);
    for (int i = t; i < P * r; i += NT) {
        const int tok = i / r, k = i % r;
        float s = 0.f;
        for (int d = 0; d < D; ++d) s += kc[tok][d] * vs[k][d];
        put(a.coef, coef0 + i, s);
    }
}

// The summarised-page count after a refresh: one thread per sequence.
__global__ void advance_summarized_kernel(const int32_t* seq_lens, const int32_t* page_begin,
                                          int32_t* summarized, int batch, int page_size,
                                          int max_pages, int max_new_pages) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= batch) return;
    int full = seq_lens[b] / page_size;
    full = full < 0 ? 0 : (full > max_pages ? max_pages : full);
    const int lo = page_begin[b];
    const int hi = lo + max_new_pages < full ? lo + max_new_pages : full;
    const int cur = summarized[b];
    if (cur >= lo && hi > cur) summarized[b] = hi;
}

template <int P, int D>
hipError_t launch_pd(const BuildParams& p, hipStream_t s) {
    const long units =
        (long)p.batch * (p.refresh_pages > 0 ? p.refresh_pages : p.max_pages) * p.num_kv_heads;
    if (units == 0) return hipSuccess;
    if (p.bf16)
        hipLaunchKernelGGL((build_kernel<P, D, true>), dim3((unsigned)units),
                           dim3(build_threads<P>()), 0, s, p);
    else
        hipLaunchKernelGGL((build_kernel<P, D, false>), dim3((unsigned)units),
                           dim3(build_threads<P>()), 0, s, p);
    return hipGetLastError();
}

}  // namespace

bool build_supported(int page_size, int head_dim, int rank) {
    return (page_size == 16 || page_size == 64) && (head_dim == 64 || head_dim == 128) &&
           rank >= 1 && rank <= 16 && rank <= page_size && rank <= head_dim;
}

hipError_t launch_advance_summarized(const int32_t* seq_lens, const int32_t* page_begin,
                                     int32_t* summarized, int32_t batch, int32_t page_size,
                                     int32_t max_pages, int32_t max_new_pages, hipStream_t s) {
    hipLaunchKernelGGL(advance_summarized_kernel, dim3((batch + 255) / 256), dim3(256), 0, s,
                       seq_lens, page_begin, summarized, batch, page_size, max_pages,
                       max_new_pages);
    return hipGetLastError();
}

hipError_t launch_build(const BuildParams& p, hipStream_t s) {
    if (p.page_size == 16 && p.head_dim == 64) return launch_pd<16, 64>(p, s);
    if (p.page_size == 16 && p.head_dim == 128) return launch_pd<16, 128>(p, s);
    if (p.page_size == 64 && p.head_dim == 64) return launch_pd<64, 64>(p, s);
    return launch_pd<64, 128>(p, s);
}

}  // namespace locks
