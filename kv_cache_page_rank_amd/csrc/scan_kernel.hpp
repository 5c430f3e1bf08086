// Kernel template of the summary scan and its launchers, instantiated once
// per stored summary type by scan_f32.hip, scan_bf16.hip and scan_q8q4.hip
// (one translation unit each, so they compile in parallel); scan.hip
// dispatches.  The per-type batch functions are in scan_batch_*.hpp, the
// shared pieces (and the method's description) in scan_common.hpp.
#pragma once

#include "scan_batch_bf16.hpp"
#include "scan_batch_f32.hpp"
#include "scan_batch_q8q4.hpp"

namespace locks {

namespace {

// Code summaries keep their per-wave tables in LDS and fit three waves per
// SIMD (asked for here, so that batches of many waves overlap one wave's
// set-up with another's tiles); the others take the registers they need.
template <typename TS, int P, int D, int RR, bool kExact, bool kHeads, bool kOff32,
          int NP = kBatch, int PF = kPrefetch>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(TS) == 1 ? 3 : 1)))
void scan_kernel(const ScanParams a) {
    static_assert(P % 16 == 0 && D % 32 == 0, "P a multiple of 16, d of 32");
    static_assert(RR == 4 || RR == 8 || RR == 16, "padded rank");
    static_assert(NP % kRunPages == 0 && NP <= kWave, "whole runs per wave");
    static_assert(sizeof(TS) == 4 || NP == kBatch, "the bf16 and code paths scan one run per wave");
    static_assert(sizeof(TS) != 2 || PF == kPrefetch, "the bf16 path keeps one tile in flight");
    constexpr int E = Summ<TS>::E;
    constexpr int NCH = D / (4 * E);

    WaveCtx<D> x;
    x.lane = threadIdx.x & 63;
    x.w = x.lane >> 4;
    x.c = x.lane & 15;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nbatch = (a.max_pages + NP - 1) / NP;
    if (wave >= a.batch * a.num_kv_heads * nbatch) return;
    const int jb = wave % nbatch;
    x.g = (wave / nbatch) % a.num_kv_heads;
    x.b = wave / (nbatch * a.num_kv_heads);
    x.Hkv = a.num_kv_heads;
    x.G = a.num_q_heads / x.Hkv;
    x.r = a.rank;
    x.head_ok = x.c < x.G;
    x.j0 = jb * NP;
    const int c = x.c, w = x.w;

    // Lane l looks after page j0 + l % NP.  Its block-table entry is read
    // together with the sequence length (clamped index, kept only if the page
    // is full), so the two loads overlap instead of following each other.
    const int pl = x.lane % NP;
    const int jc = x.j0 + pl;
    const int p_spec =
        a.block_table[(size_t)x.b * a.max_pages + (jc < a.max_pages ? jc : a.max_pages - 1)];
    // the pages that compete: full pages whose summaries exist (the count is
    // read beside the length; pages past it are not scanned and get -inf)
    const int summ_raw = a.summarized ? a.summarized[x.b] : 0;
    const int full =
        candidate_pages(a.seq_lens[x.b], summ_raw, a.summarized != nullptr, P, a.max_pages);
    // Query fragment, in the contraction order of the summary loads:
    // qf[E t + e] = q[h][4E t + E w + e] for head h = c, as loaded; the batch
    // functions scale it to log2 units (qs, 0 for padding heads) when they
    // split it, after their first summary loads are issued.  Its loads come
    // after the block-table and length reads (the compiler places them past
    // the early exit, beside the first tile's loads): vector loads complete in
    // issue order, so a wave that waits for its block-table entry would
    // otherwise wait for the query as well (measured: 0.2-0.9 us faster).
    x.qs = x.head_ok ? kLog2e / sqrtf((float)D) : 0.0f;
    {
        const float* qp =
            a.q + ((size_t)x.b * a.num_q_heads + x.g * x.G + (x.head_ok ? c : 0)) * D;
#pragma unroll
        for (int t = 0; t < NCH; ++t)
#pragma unroll
            for (int h4 = 0; h4 < E / 4; ++h4) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(qp + 4 * E * t + E * w + 4 * h4);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    x.qf[E * t + 4 * h4 + e] = v[e];
            }
    }

    x.out_page = a.page_logmass + ((size_t)x.b * x.Hkv + x.g) * a.max_pages;
    if (x.j0 >= full) {  // whole batch past the full pages
        const int nruns = (a.max_pages + kRunPages - 1) / kRunPages;
        const int run = x.j0 / kRunPages + x.lane;
        if (a.run_max && x.lane < NP / kRunPages && run < nruns)
            a.run_max[((size_t)x.b * x.Hkv + x.g) * nruns + run] = -INFINITY;
        if (x.lane < NP && x.j0 + x.lane < a.max_pages) {
            x.out_page[x.j0 + x.lane] = -INFINITY;
            if constexpr (kHeads)
                for (int hh = 0; hh < x.G; ++hh)
                    a.head_logmass[((size_t)x.b * a.num_q_heads + x.g * x.G + hh) * a.max_pages +
                                   x.j0 + x.lane] = -INFINITY;
        }
        return;
    }
    x.my_phys = (jc < full && p_spec >= 0 && p_spec < a.num_blocks) ? p_spec : -1;


    // every page of the batch present and the rank not padded: no masking
    if constexpr (kExact) {
        if (x.j0 + NP <= full && __ballot(x.lane < NP && x.my_phys < 0) == 0ull) {
            if constexpr (sizeof(TS) == 1)
                scan_batch_q<P, D, RR, kExact, kHeads, kOff32, false, PF>(a, x);
            else if constexpr (sizeof(TS) == 2)
                scan_batch_bf16<P, D, RR, kExact, kHeads, kOff32, false>(a, x);
            else
                scan_batch_f32<P, D, RR, kExact, kHeads, kOff32, false, NP, PF>(a, x);
            return;
        }
    }
    if constexpr (sizeof(TS) == 1)
        scan_batch_q<P, D, RR, kExact, kHeads, kOff32, true, PF>(a, x);
    else if constexpr (sizeof(TS) == 2)
        scan_batch_bf16<P, D, RR, kExact, kHeads, kOff32, true>(a, x);
    else
        scan_batch_f32<P, D, RR, kExact, kHeads, kOff32, true, NP, PF>(a, x);
}

template <typename TS, int P, int D, int RR, bool kHeads, bool kOff32, int NP, int PF>
hipError_t launch4(const ScanParams& p, hipStream_t s) {
    const long waves = (long)p.batch * p.num_kv_heads * ((p.max_pages + NP - 1) / NP);
    const unsigned blocks = (unsigned)((waves + 3) / 4);
    if (blocks == 0) return hipSuccess;
    if (p.rank == RR)
        hipLaunchKernelGGL((scan_kernel<TS, P, D, RR, true, kHeads, kOff32, NP, PF>),
                           dim3(blocks), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((scan_kernel<TS, P, D, RR, false, kHeads, kOff32, NP, PF>),
                           dim3(blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <typename TS, int P, int D, int RR, int NP = kBatch, int PF = kPrefetch>
hipError_t launch_ts(const ScanParams& p, hipStream_t s) {
    // largest summary array (basis or coefficients) in bytes
    size_t per_unit = (size_t)p.rank * (D > P ? D : P) * sizeof(TS);
    if (sizeof(TS) == 1) {  // codes: centroid D, basis r D/2, coefficients P r bytes
        per_unit = (size_t)p.rank * (D / 2 > P ? D / 2 : P);
        per_unit = per_unit > (size_t)D ? per_unit : (size_t)D;
    }
    const bool off32 = (size_t)p.num_blocks * p.num_kv_heads * per_unit < (size_t(1) << 32);
    if (p.head_logmass != nullptr)
        return off32 ? launch4<TS, P, D, RR, true, true, NP, PF>(p, s)
                     : launch4<TS, P, D, RR, true, false, NP, PF>(p, s);
    return off32 ? launch4<TS, P, D, RR, false, true, NP, PF>(p, s)
                 : launch4<TS, P, D, RR, false, false, NP, PF>(p, s);
}

template <typename TS, int P, int D, int RR>
hipError_t launch_typed(const ScanParams& p, hipStream_t s) {
    return launch_ts<TS, P, D, RR>(p, s);
}

template <typename TS, int P, int D>
hipError_t launch_rr(const ScanParams& p, hipStream_t s) {
    if (p.rank <= 4) return launch_typed<TS, P, D, 4>(p, s);
    if (p.rank <= 8) return launch_typed<TS, P, D, 8>(p, s);
    return launch_typed<TS, P, D, 16>(p, s);
}

// Every supported (page size, head dim) for one stored summary type.
template <typename TS>
hipError_t launch_scan_of(const ScanParams& p, hipStream_t s) {
    if (p.page_size == 16 && p.head_dim == 64) return launch_rr<TS, 16, 64>(p, s);
    if (p.page_size == 16 && p.head_dim == 128) return launch_rr<TS, 16, 128>(p, s);
    if (p.page_size == 64 && p.head_dim == 64) return launch_rr<TS, 64, 64>(p, s);
    return launch_rr<TS, 64, 128>(p, s);
}

}  // namespace

}  // namespace locks
