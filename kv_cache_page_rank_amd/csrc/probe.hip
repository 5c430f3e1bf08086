// Measurement probes: two read-only kernels that give the summary scan's
// roofline its ceilings on the device it runs on, built with the same
// compiler and flags as the scan.
//
//   stream_read_kernel   a contiguous read of a buffer, 16-byte loads, eight
//                        in flight per lane, chunks strided over the grid:
//                        what HBM delivers to a plain streaming kernel.
//   pattern_read_kernel  the bytes the fp32 summary scan reads (P 64, d 128,
//                        r 8), in the scan's access pattern: one wave per run
//                        of 16 consecutive pages of one (b, g), pages mapped
//                        through the block table, the query fragment, the 16
//                        centroids (16-byte loads), then 8 tiles of 2 pages,
//                        each 16 basis rows as 16-byte loads and the 2 pages'
//                        coefficients as 8-byte loads, one tile in flight
//                        ahead of the one consumed; one float per page is
//                        written.  The loaded words are only summed (one add
//                        per word), so the kernel shows what the scan's
//                        loads cost without its matrix and exponential work.
//
// Neither is part of the decode step.
#include "device_common.hpp"
#include "launchers.hpp"

namespace locks {

namespace {

// Each workgroup step reads a contiguous chunk of kStreamUnroll x 256 x 16
// bytes (eight 16-byte loads in flight per lane, each load instruction 1 KiB
// contiguous per wave), chunks strided over the grid.
constexpr int kStreamUnroll = 8;

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ buf,
                                                          size_t n16, float* __restrict__ sink) {
    constexpr size_t kChunk = (size_t)kStreamUnroll * 256;
    uint32_t acc = 0u;
    size_t base = (size_t)blockIdx.x * kChunk;
    const size_t step = (size_t)gridDim.x * kChunk;
    for (; base + kChunk <= n16; base += step) {
        u32x4 v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) v[u] = buf[base + (size_t)u * 256 + threadIdx.x];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) acc += (v[u][0] ^ v[u][1]) + (v[u][2] ^ v[u][3]);
    }
    // the tail that does not fill a chunk
    for (size_t i = base + threadIdx.x; base < n16 && i < n16; i += 256) {
        const u32x4 a = buf[i];
        acc += a[0] + a[1] + a[2] + a[3];
    }
    // one value per wave (written whatever the sum, so the loads stay live)
    acc += __shfl_xor(acc, 1, kWave);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = (float)acc;
}

constexpr int kP = 64, kD = 128, kR = 8;
constexpr int kPagesPerWave = kRunPages;  // 16
constexpr int kTilePages = 2;             // 16 basis rows = 2 pages x 8 rows
constexpr int kTiles = kPagesPerWave / kTilePages;

struct PatternTile {
    u32x4 v[kD / 16];                 // 8 x 16 bytes of one basis row
    u32x2 cf[kTilePages][kP / 16];    // 2 pages x 4 token tiles x 8 bytes
};

__global__ __launch_bounds__(256) void pattern_read_kernel(const ProbeScanParams a) {
    const int lane = threadIdx.x & 63, w = lane >> 4, c = lane & 15;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nruns = (a.max_pages + kPagesPerWave - 1) / kPagesPerWave;
    if (wave >= a.batch * a.num_kv_heads * nruns) return;
    const int jb = wave % nruns;
    const int g = (wave / nruns) % a.num_kv_heads;
    const int b = wave / (nruns * a.num_kv_heads);
    const int Hkv = a.num_kv_heads, G = a.num_q_heads / Hkv;
    const int j0 = jb * kPagesPerWave;
    int full = a.seq_lens[b] / kP;
    full = full < 0 ? 0 : (full > a.max_pages ? a.max_pages : full);
    const int jc = j0 + c;
    const int p_spec = a.block_table[(size_t)b * a.max_pages + (jc < a.max_pages ? jc : a.max_pages - 1)];
    float* out = a.page_out + ((size_t)b * Hkv + g) * a.max_pages;
    if (j0 >= full) {
        if (w == 0 && jc < a.max_pages) out[jc] = -INFINITY;
        return;
    }
    // pages that are not full read block 0 (a valid address); every page of
    // the 1M-token and 128K-token layers is full, so their bytes are exact
    const int my_phys = (jc < full && p_spec >= 0 && p_spec < a.num_blocks) ? p_spec : 0;
    const uint32_t* basis = static_cast<const uint32_t*>(a.basis);
    const uint32_t* coef = static_cast<const uint32_t*>(a.coef);
    const uint32_t* mu = static_cast<const uint32_t*>(a.mu);

    float acc = 0.0f;
    auto eat4 = [&](const u32x4& v) {
        acc += __uint_as_float(v[0]) + __uint_as_float(v[1]) + __uint_as_float(v[2]) +
               __uint_as_float(v[3]);
    };
    // query fragment of head c (head 0 for padding heads)
    const float* qp = a.q + ((size_t)b * a.num_q_heads + g * G + (c < G ? c : 0)) * kD;
    u32x4 qv[kD / 16];
#pragma unroll
    for (int t = 0; t < kD / 16; ++t) qv[t] = *reinterpret_cast<const u32x4*>(qp + 16 * t + 4 * w);

    auto load_tile = [&](int tt, PatternTile& T) {
        const int pin = (c & 3) / 2, kk = 2 * (c >> 2) + ((c & 3) % 2);  // the scan's row order
        const int pj = __shfl(my_phys, tt * kTilePages + pin, kWave);
        const uint32_t* src = basis + (((size_t)pj * Hkv + g) * kR + kk) * kD + 4 * w;
#pragma unroll
        for (int t = 0; t < kD / 16; ++t) T.v[t] = *reinterpret_cast<const u32x4*>(src + 16 * t);
#pragma unroll
        for (int p = 0; p < kTilePages; ++p) {
            const int pp = __builtin_amdgcn_readlane(my_phys, tt * kTilePages + p);
            const uint32_t* cs = coef + ((size_t)pp * Hkv + g) * kP * kR;
#pragma unroll
            for (int mt = 0; mt < kP / 16; ++mt)
                T.cf[p][mt] = *reinterpret_cast<const u32x2*>(cs + (16 * mt + c) * kR + 2 * w);
        }
    };
    PatternTile ring[2];
    load_tile(0, ring[0]);
    {
        const uint32_t* src = mu + ((size_t)my_phys * Hkv + g) * kD + 4 * w;
        u32x4 mv[kD / 16];
#pragma unroll
        for (int t = 0; t < kD / 16; ++t) mv[t] = *reinterpret_cast<const u32x4*>(src + 16 * t);
#pragma unroll
        for (int t = 0; t < kD / 16; ++t) {
            eat4(mv[t]);
            eat4(qv[t]);
        }
    }
#pragma unroll
    for (int tt = 0; tt < kTiles; ++tt) {
        if (tt + 1 < kTiles) load_tile(tt + 1, ring[(tt + 1) & 1]);
        const PatternTile& cur = ring[tt & 1];
#pragma unroll
        for (int t = 0; t < kD / 16; ++t) eat4(cur.v[t]);
#pragma unroll
        for (int p = 0; p < kTilePages; ++p)
#pragma unroll
            for (int mt = 0; mt < kP / 16; ++mt)
                acc += __uint_as_float(cur.cf[p][mt][0]) + __uint_as_float(cur.cf[p][mt][1]);
#pragma unroll
        for (int p = 0; p < kTilePages; ++p) {
            const int pb = tt * kTilePages + p;
            if (w == (pb >> 2) && c == 0 && j0 + pb < a.max_pages) out[j0 + pb] = acc;
        }
    }
}

}  // namespace

hipError_t launch_probe_stream(const void* buf, size_t bytes, float* sink, int32_t blocks,
                               hipStream_t s) {
    hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, s,
                       static_cast<const u32x4*>(buf), bytes / 16, sink);
    return hipGetLastError();
}

bool probe_scan_supported(int page_size, int head_dim, int rank) {
    return page_size == kP && head_dim == kD && rank == kR;
}

hipError_t launch_probe_scan(const ProbeScanParams& p, hipStream_t s) {
    const long waves = (long)p.batch * p.num_kv_heads * ((p.max_pages + kPagesPerWave - 1) / kPagesPerWave);
    const unsigned blocks = (unsigned)((waves + 3) / 4);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(pattern_read_kernel, dim3(blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace locks
